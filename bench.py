"""Benchmark of the quantized paged-KV decode path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--quick]

Headline: the Llama-3-8B-shaped INT8 workload (64 sequences, lengths U[512,
4096], 32 query / 8 KV heads, head dim 128, per-tensor absmax scales).  One step
writes the new token of every sequence into the paged cache (kvq_cache_write)
and runs the paged decode (kvq_paged_attention_decode: balanced chunks of the
concatenated page list, then the split-KV merge kernel).  The page pool is replicated R times
(>= 1.5 GB in total) and step s uses copy s % R, so the 256 MB Infinity Cache
cannot serve the pages from a previous step; inputs are resident in HBM before
the timed region.

value = algorithmic KV bytes read per step / step time (GB/s), where the KV bytes
are sum_b L_b * Hkv * (K + V bytes per token-head: 2*D for 8-bit codes).
The JSON line also carries the decode kernel's roofline, per-dtype decode
figures for the other workloads, cache-write / convert / calibrate GB/s, and the
oracle's CPU throughput on a bounded sample.  Beside each decode it times a
launch that reads the same pages and computes nothing (read_only, from
lib/libkvq_probe.so): what one launch reaches on those pages.
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

HBM_PEAK_GBS = 8000.0
MALL_DEFEAT_BYTES = 1.5e9


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline only (no per-dtype lines)")
    ap.add_argument("--only", default=None, help="comma list of per-dtype workloads to run")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 5 device-to-device copies of BYTES bytes (calibrates HBM byte counters)")
    ap.add_argument("--trace-summary", nargs=3, metavar=("STATS_CSV", "OUT", "COMMAND"),
                    help="write the text summary of a rocprofv3 --kernel-trace --stats csv run and exit")
    ap.add_argument("--counter-summary", nargs=4, metavar=("CSV_A", "CSV_B", "OUT", "COMMAND"),
                    help="write per-page instruction and wait counters of the chunk kernels (headline decode "
                         "and 16-token verify) from two rocprofv3 --pmc runs")
    ap.add_argument("--traffic-summary", nargs=8,
                    metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "COPY_BYTES",
                             "OUT", "COMMAND"),
                    help="write HBM bytes per decode call of WORKLOAD from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "runs of --profile-workload WORKLOAD and of the copy probe, and exit")
    ap.add_argument("--profile-workload", default=None, metavar="NAME",
                    help="only build workload NAME and run its decode calls (for rocprofv3 runs of one workload)")
    return ap.parse_args()


def trace_summary(stats_csv, out, command):
    """Text summary of rocprofv3 kernel statistics (durations in microseconds)."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["rocprofv3 kernel-trace summary", "", "command:", "  " + command, "",
             "kvq_paged_attention_decode source hash: " + decode_source_hash(), "",
             f"{'kernel':<64} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for r in rows:
        name = r["Name"].replace("void ", "").replace("kvq::(anonymous namespace)::", "")
        name = name.split("(")[0] if "kvq::" in r["Name"] else name[:64]
        lines.append(f"{name[:64]:<64} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                     f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} {float(r['Percentage']):>6.1f}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counter_summary(csv_a, csv_b, out, command):
    """SQ counters of decode_chunk_kernel per 16-token page and KV head (the sum over
    the waves that read it), averaged over dispatches.  Each kernel instantiation is
    matched to the workload of the same element formats, head size and query-token
    count among those bench.py times (llama8b_int8 and another on the same formats
    with several query tokens: verify16_int8)."""
    import csv
    import re
    from workloads import WORKLOADS, make_decode_inputs
    from quantized_paged_kv_absmax_amd import _lib
    names = ["llama8b_int8", "verify16_int8", "fp8_e4m3", "int4", "int4_had", "bf16"]
    kernels, pages = {}, {}
    for wl in names:
        w = WORKLOADS[wl]
        kt = _lib.INT4_HAD if w.k_dtype == "int4h" else _lib.DTYPES[w.k_dtype]
        key = (kt, _lib.DTYPES[w.v_dtype], w.D, w.n_q > 1)
        kernels.setdefault(key, wl)
    per, seen = {}, []  # workload -> counter -> per-page value
    for path in (csv_a, csv_b):
        tot, disp = {}, {}
        for r in csv.DictReader(open(path)):
            m = re.search(r"decode_chunk_kernel<(-?\d+), (-?\d+), (\d+), \d+, (true|false)", r["Kernel_Name"])
            if m is None:
                continue
            wl = kernels.get((int(m.group(1)), int(m.group(2)), int(m.group(3)), m.group(4) == "true"))
            if wl is None:
                continue
            if wl not in pages:
                w = WORKLOADS[wl]
                inp = make_decode_inputs(w)
                pages[wl] = int(((inp.seq_lens.astype(np.int64) + 15) // 16).sum()) * w.Hkv
                seen.append(wl)
            c = r["Counter_Name"].replace("SQ_", "")
            tot.setdefault(wl, {})
            tot[wl][c] = tot[wl].get(c, 0.0) + float(r["Counter_Value"])
            disp.setdefault(wl, set()).add(r["Dispatch_Id"])
        for wl, vals in tot.items():
            for c, v in vals.items():
                per.setdefault(wl, {})[c] = v / len(disp[wl]) / pages[wl]
    lines = ["rocprofv3 SQ counters of decode_chunk_kernel per 16-token page and KV head", "", "command:",
             "  " + command, "", "kvq_paged_attention_decode source hash: " + decode_source_hash(), "",
             "Summed over the waves that read a page (the several-token kernel runs four, one per",
             "16-column tile); *_CYCLES, ACTIVE_* and WAIT_* in the counters' own units.", ""]
    for wl in seen:
        lines.append(f"{wl}: {pages[wl]} page-heads per call")
        for c, v in sorted(per.get(wl, {}).items()):
            lines.append(f"  {c:<28} {v:10.1f}")
        lines.append("")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_summary(workload, fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes, out, command):
    """HBM bytes per decode call (chunk + reduce kernels) from FETCH_SIZE / WRITE_SIZE,
    each scaled by what the same counter reads for a copy of known size."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            k = r["Kernel_Name"]
            d = acc.setdefault(k, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"]) * 1024.0   # KiB
        return acc

    def avg(acc, key):
        vals = [v for k, d in acc.items() if key in k for v in d.values()]
        return (sum(vals) / len(vals), len(vals)) if vals else (0.0, 0)

    copy_bytes = float(copy_bytes)
    cf, _ = avg(per_kernel(cfetch_csv, "FETCH_SIZE"), "copyBuffer")
    cw, _ = avg(per_kernel(cwrite_csv, "WRITE_SIZE"), "copyBuffer")
    if cf == 0.0:
        cf, _ = avg(per_kernel(cfetch_csv, "FETCH_SIZE"), "")
        cw, _ = avg(per_kernel(cwrite_csv, "WRITE_SIZE"), "")
    f_scale, w_scale = copy_bytes / cf, copy_bytes / cw
    fetch, wr = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    cf_chunk, n = avg(fetch, "decode_chunk_kernel")
    cf_red, _ = avg(fetch, "decode_reduce")
    cw_chunk, _ = avg(wr, "decode_chunk_kernel")
    cw_red, _ = avg(wr, "decode_reduce")
    total = (cf_chunk + cf_red) * f_scale + (cw_chunk + cw_red) * w_scale
    from workloads import WORKLOADS, make_decode_inputs
    alg = kv_bytes(make_decode_inputs(WORKLOADS[workload]))
    lines = [f"rocprofv3 HBM traffic of one kvq_paged_attention_decode call ({workload} workload)", "",
             "command:", "  " + command, "",
             f"kernel_source_hash: {decode_source_hash()}",
             f"copy_probe_bytes: {copy_bytes:.0f}",
             f"fetch_scale (copy bytes / copy FETCH_SIZE bytes): {f_scale:.4f}",
             f"write_scale (copy bytes / copy WRITE_SIZE bytes): {w_scale:.4f}",
             f"decode_chunk_kernel dispatches: {n}",
             f"decode_chunk_kernel fetch_bytes (scaled): {cf_chunk * f_scale:.0f}",
             f"decode_chunk_kernel write_bytes (scaled): {cw_chunk * w_scale:.0f}",
             f"decode_reduce_kernel fetch_bytes (scaled): {cf_red * f_scale:.0f}",
             f"decode_reduce_kernel write_bytes (scaled): {cw_red * w_scale:.0f}",
             f"algorithmic_kv_bytes: {alg}",
             f"traffic_over_algorithmic: {total / alg:.4f}",
             f"hbm_bytes_per_launch: {total:.0f}"]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_probe(nbytes):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch scale the
    counters read on the decode kernel to bytes."""
    import torch
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "dispatches": 5}))


# bytes one (token, KV head) row of K or V occupies: codes, plus the float32
# (scale, zero point) pair of INT4
ROW_BYTES = {"bf16": lambda D: 2 * D, "int8": lambda D: D, "e4m3": lambda D: D, "e5m2": lambda D: D,
             "int4": lambda D: D // 2 + 8, "int4h": lambda D: D // 2 + 8}


def kv_bytes(inp):
    """Algorithmic KV bytes one decode reads: sum_b L_b * Hkv * (K row + V row)."""
    w = inp.w
    per = ROW_BYTES[w.k_dtype](w.D) + ROW_BYTES[w.v_dtype](w.D)
    return int(inp.seq_lens.astype(np.int64).sum()) * w.Hkv * per


def decode_source_hash():
    """Hash of the decode kernels' source with comments and blank space removed, so
    that a profile stays matched to its kernel across edits of comments only."""
    import re
    h = hashlib.sha256()
    for f in ("decode_kernel.h", "decode.hip", "kvq_device.h", "kvq_rows.h"):
        text = open(os.path.join(ROOT, "quantized_paged_kv_absmax_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload, kernel_hash):
    """HBM bytes per decode launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class GpuWorkload:
    """A workload's cache on the GPU, replicated for rotation, plus its step inputs."""

    def __init__(self, name, device, rotate=True):
        import torch
        import quantized_paged_kv_absmax_amd as kvq
        from workloads import WORKLOADS, make_decode_inputs, make_calibration_set, scatter_rows_to_pages

        self.torch, self.kvq = torch, kvq
        w = WORKLOADS[name]
        self.name, self.w = name, w
        t0 = time.perf_counter()
        inp = make_decode_inputs(w)
        self.inp = inp
        self.gen_s = time.perf_counter() - t0

        def t16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

        c = kvq.PagedKVCache(inp.num_blocks, w.Hkv, w.D, w.k_dtype, w.v_dtype, k_gran=w.k_gran, v_gran=w.v_gran,
                             device=device)
        self.cache = c
        self.extra = {}
        qmax = {"int8": "int8", "e4m3": "e4m3", "e5m2": "e5m2"}
        ck, cv = make_calibration_set(w, inp)
        if w.k_scale_mode == "absmax" and w.k_dtype in qmax:
            xk = t16(ck)
            self.extra["calibrate_gbs"] = self._time_calibrate(xk, w.k_gran, w.k_dtype, c)
            kvq.kvq_calibrate_scales(xk, w.k_gran, w.k_dtype, c.k_absmax, c.k_scale)
            del xk
        if w.v_scale_mode == "absmax" and w.v_dtype in qmax:
            kvq.kvq_calibrate_scales(t16(cv), w.v_gran, w.v_dtype, c.v_absmax, c.v_scale)
        mask = inp.prompt_mask()
        new_idx = np.nonzero(~mask)[0]
        if w.from_bf16_cache:
            kp = t16(scatter_rows_to_pages(inp.k_bits, inp.slot_mapping, inp.num_blocks))
            vp = t16(scatter_rows_to_pages(inp.v_bits, inp.slot_mapping, inp.num_blocks))
            self.extra["convert"] = self._time_convert(kp, vp)
            kvq.kvq_convert_cache(c, kp, vp)
            del kp, vp
        else:
            pidx = np.nonzero(mask)[0]
            kd, vd = t16(inp.k_bits[pidx]), t16(inp.v_bits[pidx])
            sl = torch.from_numpy(inp.slot_mapping[pidx]).to(device)
            self.extra["bulk_write"] = self._time_write(kd, vd, sl)
            kvq.kvq_cache_write(c, kd, vd, sl)
            del kd, vd, sl
        # the decode step's own tokens (written inside the step)
        self.k_new = t16(inp.k_bits[new_idx]) if new_idx.size else None
        self.v_new = t16(inp.v_bits[new_idx]) if new_idx.size else None
        self.slot_new = torch.from_numpy(inp.slot_mapping[new_idx]).to(device) if new_idx.size else None
        if self.k_new is not None:
            kvq.kvq_cache_write(c, self.k_new, self.v_new, self.slot_new)
        torch.cuda.synchronize()
        self.q = t16(inp.q_bits)
        self.bt = torch.from_numpy(inp.block_tables).to(device)
        self.sl = torch.from_numpy(inp.seq_lens).to(device)
        self.sm = float(np.float32(1.0) / np.sqrt(np.float32(w.D)))
        pool_bytes = c.k_pages.numel() + c.v_pages.numel() + (0 if c.k_meta is None else 8 * c.k_meta.numel())
        self.R = max(2, int(np.ceil(MALL_DEFEAT_BYTES / pool_bytes))) if rotate else 1
        self.copies = [(c.k_pages, c.v_pages, c.k_meta, c.v_meta)]
        for _ in range(self.R - 1):
            self.copies.append(tuple(None if t is None else t.clone() for t in self.copies[0]))
        self.structs = []
        for kp, vp, km, vm in self.copies:
            s = c.struct(kp, vp)
            if km is not None:
                s.k_meta, s.v_meta = km.data_ptr(), vm.data_ptr()
            self.structs.append(s)
        ws = kvq.kvq_verify_workspace_size(w.B, w.n_q, w.Hq, w.Hkv, w.D, inp.max_seq_len, w.partition)
        self.ws = torch.zeros(max(ws, 16), dtype=torch.uint8, device=device)
        self.out = torch.empty((w.B * w.n_q, w.Hq, w.D), dtype=torch.bfloat16, device=device)
        self.kv_bytes = kv_bytes(inp)
        torch.cuda.synchronize()

    # ---- pieces of the step ----
    def write_new(self, i):
        if self.k_new is not None:
            self.kvq.kvq_cache_write(self.cache, self.k_new, self.v_new, self.slot_new, struct=self.structs[i % self.R])

    def fused_step_ok(self):
        """One new token per sequence and one query token: the step fits one call."""
        return self.k_new is not None and self.w.n_q == 1 and self.k_new.shape[0] == self.w.B

    def write_and_decode(self, i):
        """The step in one call (the new token's write inside the decode launch)."""
        self.kvq.kvq_paged_attention_decode_write(self.cache, self.k_new, self.v_new, self.slot_new, self.q, self.bt,
                                                  self.sl, self.inp.max_seq_len, self.sm, partition=self.w.partition,
                                                  workspace=self.ws, out=self.out, struct=self.structs[i % self.R])

    def decode(self, i):
        if self.w.n_q > 1:
            self.kvq.kvq_paged_attention_verify(self.cache, self.q, self.w.n_q, self.bt, self.sl, self.inp.max_seq_len,
                                                self.sm, partition=self.w.partition, workspace=self.ws, out=self.out,
                                                struct=self.structs[i % self.R])
            return
        self.kvq.kvq_paged_attention_decode(self.cache, self.q, self.bt, self.sl, self.inp.max_seq_len, self.sm,
                                            partition=self.w.partition, workspace=self.ws, out=self.out,
                                            struct=self.structs[i % self.R])

    # ---- timers for the set-up kernels (reported as extra figures) ----
    def _events(self, fn, reps):
        torch = self.torch
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    def _time_write(self, kd, vd, sl):
        c, kvq = self.cache, self.kvq
        scratch = kvq.PagedKVCache(c.num_blocks, c.num_kv_heads, c.head_dim, c.k_dtype, c.v_dtype,
                                   k_gran=c.k_gran, v_gran=c.v_gran, device=kd.device)
        t = self._events(lambda: kvq.kvq_cache_write(scratch, kd, vd, sl), 5)
        T, H, D = kd.shape
        rb = {0: 2 * D, 1: D, 2: D, 3: D, 4: D // 2 + 8}
        moved = T * H * (2 * 2 * D) + T * H * (rb[c.k_dtype] + rb[c.v_dtype])
        del scratch
        return {"tokens": int(T), "us": t * 1e6, "gbs": moved / t / 1e9}

    def _time_convert(self, kp, vp):
        c, kvq = self.cache, self.kvq
        t = self._events(lambda: kvq.kvq_convert_cache(c, kp, vp), 5)
        n = kp.numel()
        moved = 2 * n * 2 + 2 * (n // 2 + (n // c.head_dim) * 8)
        return {"blocks": c.num_blocks, "us": t * 1e6, "gbs": moved / t / 1e9}

    def _time_calibrate(self, x, gran, dt, c):
        torch, kvq = self.torch, self.kvq
        a = torch.zeros_like(c.k_absmax)
        s = torch.zeros_like(c.k_scale)
        t = self._events(lambda: kvq.kvq_calibrate_scales(x, gran, dt, a, s), 5)
        return {"tokens": int(x.shape[0]), "us": t * 1e6, "gbs": x.numel() * 2 / t / 1e9}


def time_steps(gw, steps, warmup, with_write=True, fused=True):
    """Warmup, then K timed steps (write + decode) bracketed by synchronize and
    one event pair; returns ms per step.  fused: the step as one call
    (kvq_paged_attention_decode_write) where it fits, else the write and the decode."""
    torch = gw.torch
    one = with_write and fused and gw.fused_step_ok()

    def step(i):
        if one:
            gw.write_and_decode(i)
            return
        if with_write:
            gw.write_new(i)
        gw.decode(i)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_decode_calls(gw, samples=60, batch=10, warmup=5):
    """The decode call alone, on the stream the library launches on (torch's
    current stream): ``samples`` event pairs, each around ``batch`` calls launched
    back to back (rotating pool copies), so that the per-call figure holds the
    kernels and the gaps between them but not an event's own launch latency.
    Also ``samples`` single calls each between its own event pair (that latency
    included).  Returns per-call microseconds: (batched samples, single samples)."""
    torch = gw.torch
    for i in range(warmup):
        gw.decode(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    k = 0
    for a, b in ev:
        a.record()
        for _ in range(batch):
            gw.decode(k)
            k += 1
        b.record()
    torch.cuda.synchronize()
    batched = np.array([a.elapsed_time(b) * 1e3 / batch for a, b in ev])
    ev1 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    for a, b in ev1:
        a.record()
        gw.decode(k)
        k += 1
        b.record()
    torch.cuda.synchronize()
    single = np.array([a.elapsed_time(b) * 1e3 for a, b in ev1])
    return batched, single


def page_list(inp):
    """Block ids of every page a decode reads, sequence by sequence (the order of
    the decode's concatenated page list)."""
    L = inp.seq_lens.astype(np.int64)
    ids = [inp.block_tables[b, :(L[b] + 15) // 16] for b in range(len(L)) if L[b] > 0]
    return np.concatenate(ids).astype(np.int32)


_PROBE = []


def _probe_fn():
    """kvq_probe_read_pages from lib/libkvq_probe.so (built beside libkvq.so)."""
    if not _PROBE:
        import ctypes
        lib = ctypes.CDLL(os.path.join(ROOT, "quantized_paged_kv_absmax_amd", "lib", "libkvq_probe.so"))
        f = lib.kvq_probe_read_pages
        P = ctypes.c_void_p
        f.argtypes = [P, P, P, P, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                      P, P]
        f.restype = ctypes.c_int
        _PROBE.append(f)
    return _PROBE[0]


def time_read_only(gw, samples=60, batch=10):
    """The same pages a decode call reads (K, V and INT4 metadata of each (page, KV
    head)), read by one launch of a kernel that computes nothing
    (libkvq_probe.so), in about the decode's number of waves (2048, a contiguous
    run of the page list each) and timed as time_decode_calls times the decode.
    Returns per-launch microseconds (batched samples)."""
    torch = gw.torch
    f = _probe_fn()
    c, w = gw.cache, gw.w
    lst = torch.from_numpy(page_list(gw.inp)).to(c.k_pages.device)
    page_bytes = c.k_pages[0, 0].numel()
    assert c.v_pages[0, 0].numel() == page_bytes, "K and V pages of one size"
    n_chunks = -(-2048 // w.Hkv)
    sink = torch.zeros(n_chunks * w.Hkv, dtype=torch.int32, device=c.k_pages.device)
    stream = torch.cuda.current_stream().cuda_stream

    def launch(i):
        kp, vp, km, vm = gw.copies[i % gw.R]
        st = f(kp.data_ptr(), vp.data_ptr(), None if km is None else km.data_ptr(),
               None if vm is None else vm.data_ptr(), lst.data_ptr(), lst.numel(), w.Hkv, page_bytes, n_chunks,
               c.num_blocks, sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"kvq_probe_read_pages: hipError {st}")

    for i in range(5):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    k = 0
    for a, b in ev:
        a.record()
        for _ in range(batch):
            launch(k)
            k += 1
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 / batch for a, b in ev])


def call_stats(gw, batched, single, traffic=None, read_only=None):
    med = float(np.median(batched))
    gbs = gw.kv_bytes / (med * 1e-6) / 1e9
    d = {"decode_us": med, "decode_us_p10_p90": [float(np.percentile(batched, 10)), float(np.percentile(batched, 90))],
         "decode_gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "kv_mb": gw.kv_bytes / 1e6,
         "single_call_us": float(np.median(single)), "samples": f"{len(batched)} x 10 calls"}
    if traffic is not None:
        d["traffic_bytes"] = traffic
        d["traffic_over_algorithmic"] = traffic / gw.kv_bytes
    if read_only is not None:
        r = float(np.median(read_only))
        d["read_only_us"] = r
        d["read_only_gbs"] = gw.kv_bytes / (r * 1e-6) / 1e9
        d["decode_over_read_only"] = r / med
    return d


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(min_s=8.0):
    """The oracle's decode on host cores over a bounded sample of the headline
    workload: whole passes over its sequences, one sequence at a time, until min_s
    of wall time, first with every BLAS thread the host gives, then with one."""
    import threadpoolctl
    from oracle import attention as oa
    from oracle import cache as oc
    from workloads import WORKLOADS, make_decode_inputs, make_calibration_set

    w = WORKLOADS["llama8b_int8"]
    inp = make_decode_inputs(w)
    ck, cv = make_calibration_set(w, inp)
    _, ks = oc.calibrate(ck, "per_tensor", 127.0)
    _, vs = oc.calibrate(cv, "per_tensor", 127.0)
    cache = oc.PagedCache(inp.num_blocks, w.Hkv, w.D, "int8", "int8", k_scale=ks, v_scale=vs)
    cache.write(inp.k_bits, inp.v_bits, inp.slot_mapping)
    sm = float(np.float32(1.0) / np.sqrt(np.float32(w.D)))

    def run():
        done, nbytes = 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min_s:
            b = done % w.B
            oa.decode(cache, inp.q_bits, inp.block_tables, inp.seq_lens, sm, seqs=[b])
            nbytes += int(inp.seq_lens[b]) * w.Hkv * 2 * w.D
            done += 1
        return done, nbytes, time.perf_counter() - t0

    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    done, nbytes, dt = run()
    with threadpoolctl.threadpool_limits(1):
        done1, nbytes1, dt1 = run()
    try:
        affinity = sorted(os.sched_getaffinity(0))
    except AttributeError:
        affinity = []
    aff = f"{len(affinity)} cpus ({affinity[0]}-{affinity[-1]})" if affinity else "unknown"
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "one_thread_gbs": nbytes1 / dt1 / 1e9,
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(), "affinity": aff,
            "write_calibrate_convert": oracle_write_rates(w, inp),
            "sample": f"oracle fp64 decode, one sequence at a time, of {done} sequence decodes "
                      f"({done / w.B:.2f} passes over the {w.B} sequences of the llama8b_int8 workload; "
                      f"{nbytes / 1e6:.1f} MB of int8 KV in {dt:.1f} s) with {threads} BLAS threads, then "
                      f"{done1} sequence decodes ({nbytes1 / 1e6:.1f} MB in {dt1:.1f} s) with one thread"}


def oracle_write_rates(w, inp, n_tok=32768):
    """The oracle's calibration, cache write and INT4 conversion on host cores,
    over the first n_tok tokens of the headline workload, in GB/s of the bytes
    each moves (bf16 read; codes and INT4 metadata written)."""
    from oracle import cache as oc
    k, v = inp.k_bits[:n_tok], inp.v_bits[:n_tok]
    th = n_tok * w.Hkv
    out = {"tokens": n_tok}
    t0 = time.perf_counter()
    _, ks = oc.calibrate(k, "per_tensor", 127.0)
    _, vs = oc.calibrate(v, "per_tensor", 127.0)
    out["calibrate_gbs"] = 2 * th * 2 * w.D / (time.perf_counter() - t0) / 1e9
    nb = (n_tok + 15) // 16
    slots = np.arange(n_tok, dtype=np.int64)
    cache = oc.PagedCache(nb, w.Hkv, w.D, "int8", "int8", k_scale=ks, v_scale=vs)
    t0 = time.perf_counter()
    cache.write(k, v, slots)
    out["write_int8_gbs"] = th * (2 * 2 * w.D + 2 * w.D) / (time.perf_counter() - t0) / 1e9
    src_k = np.ascontiguousarray(k.reshape(nb, 16, w.Hkv, w.D).transpose(0, 2, 1, 3))
    src_v = np.ascontiguousarray(v.reshape(nb, 16, w.Hkv, w.D).transpose(0, 2, 1, 3))
    c4 = oc.PagedCache(nb, w.Hkv, w.D, "int4", "int4")
    t0 = time.perf_counter()
    c4.convert_from_bf16(src_k, src_v, 0, nb)
    out["convert_int4_gbs"] = th * (2 * 2 * w.D + 2 * (w.D // 2 + 8)) / (time.perf_counter() - t0) / 1e9
    return out


def profile_workload(name):
    """One workload's decode calls alone (no headline), for a rocprofv3 run whose
    per-kernel figures then belong to that workload only.  "<workload>:step": its
    decode step instead (the one call that writes the new token and decodes)."""
    import torch
    import quantized_paged_kv_absmax_amd as kvq
    kvq.load()
    torch.cuda.set_device(0)
    name, _, mode = name.partition(":")
    gw = GpuWorkload(name, "cuda:0")
    if mode == "step":
        if not gw.fused_step_ok():
            raise SystemExit(f"{name}: its step is not one call")
        ms = time_steps(gw, 110, 5, with_write=True)
        print(json.dumps({"profile_workload": name + ":step", "ms_per_step": ms, "calls": 115}))
        return
    batched, single = time_decode_calls(gw, samples=10)
    d = call_stats(gw, batched, single)
    print(json.dumps({"profile_workload": name, "decode_us": d["decode_us"], "decode_gbs": d["decode_gbs"],
                      "kv_bytes": gw.kv_bytes, "calls": 10 * 10 + 10 + 5}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only: the decode path runs on a single MI355X; "
                                   "run with --gpus 1"}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.counter_summary:
        counter_summary(*args.counter_summary)
        return
    if args.profile_workload:
        profile_workload(args.profile_workload)
        return
    import torch
    import quantized_paged_kv_absmax_amd as kvq
    kvq.load()
    device = "cuda:0"
    torch.cuda.set_device(0)

    gw = GpuWorkload("llama8b_int8", device)
    print(f"[bench] llama8b_int8 ready: {gw.inp.seq_lens.sum()} tokens, KV {gw.kv_bytes / 1e6:.1f} MB, "
          f"R={gw.R} rotating copies (gen {gw.gen_s:.1f}s)", file=sys.stderr, flush=True)
    ms_step = time_steps(gw, args.steps, args.warmup, with_write=True)
    value = gw.kv_bytes / (ms_step * 1e-3) / 1e9
    # the same step as two calls (the write kernel, then the decode), for reference
    ms_two = time_steps(gw, args.steps, args.warmup, with_write=True, fused=False)
    khash = decode_source_hash()
    traffic = read_traffic("llama8b_int8", khash)
    batched, single = time_decode_calls(gw)
    head = call_stats(gw, batched, single, traffic, time_read_only(gw))
    achieved = head["decode_gbs"]
    # write alone: the 1-token-per-sequence cache write of the step
    wt = gw._events(lambda: gw.write_new(0), 50)
    per_dtype = {"int8 (llama8b_int8)": head}
    extras = {"llama8b_int8": dict(gw.extra, step_write_us=wt * 1e6,
                                   step="one call: kvq_paged_attention_decode_write" if gw.fused_step_ok()
                                   else "kvq_cache_write + kvq_paged_attention_decode",
                                   step_two_calls_ms=ms_two)}
    del gw
    torch.cuda.empty_cache()

    if not args.quick:
        names = ["fp8_e4m3", "fp8_e4m3_s1", "fp8_e5m2", "fp8_hybrid", "fp8_e4m3_head", "fp8_e5m2_cal", "bf16", "int4",
                 "int4_had", "longctx_int8", "verify16_int8"]
        if args.only:
            names = [n for n in args.only.split(",") if n]
        for name in names:
            g2 = GpuWorkload(name, device)
            samples = 20 if name == "longctx_int8" else 40
            b2, s2 = time_decode_calls(g2, samples=samples)
            d = call_stats(g2, b2, s2, read_traffic(name, khash), time_read_only(g2, samples=samples))
            per_dtype[f"{g2.w.k_dtype}/{g2.w.v_dtype} ({name})"] = d
            extras[name] = g2.extra
            print(f"[bench] {name}: decode {d['decode_us']:.1f} us, {d['decode_gbs']:.0f} GB/s", file=sys.stderr,
                  flush=True)
            del g2
            torch.cuda.empty_cache()

    # capacity: Llama-3-8B's cache (32 layers, 8 KV heads, head_dim 128) in 240 GiB of HBM
    cap_budget = 240 << 30
    cap = {d: kvq.kvq_blocks_in_budget(cap_budget, d, d, 8, 128, 32) for d in ("bf16", "int8", "e4m3", "int4")}
    extras["capacity_llama3_8b_240GiB"] = {"blocks": cap, "tokens": {d: 16 * n for d, n in cap.items()},
                                           "ratio_vs_bf16": {d: round(n / cap["bf16"], 4) for d, n in cap.items()}}
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    w = WORKLOADS_DESC
    line = {
        "metric": "paged-decode effective KV GB/s (% of 8 TB/s HBM) per KV dtype; cache-write GB/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": w,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "kvq_paged_attention_decode call: decode_chunk_kernel<INT8,INT8,128> + "
                               "decode_reduce_kernel<128>",
                     "timing": "median over 60 event pairs, each around 10 back-to-back calls on the launch "
                               "stream (p10/p90 in per_dtype)",
                     "note": "the paged decode alone (kvq_paged_attention_decode); value and ms_per_step time "
                             "the whole step, the new token's write included (extra.llama8b_int8.step)",
                     "read_only": {"us": round(head["read_only_us"], 2), "gbs": round(head["read_only_gbs"], 1),
                                   "frac": round(head["read_only_gbs"] / HBM_PEAK_GBS, 4),
                                   "decode_over_read_only": round(head["decode_over_read_only"], 4),
                                   "what": "the same pages read by one launch of a kernel that computes nothing "
                                           "(lib/libkvq_probe.so), 2048 waves, timed like the decode call"},
                     "kernel_source_hash": khash},
        "cpu_baseline": cpu,
        "per_dtype": per_dtype,
        "extra": extras,
    }
    print(json.dumps(line))


WORKLOADS_DESC = {
    "workload": "llama8b_int8: single-layer decode step (write 1 new token per sequence + paged decode, one "
                "kvq_paged_attention_decode_write call), Llama-3-8B attention shape, INT8 KV with per-tensor absmax "
                "scales",
    "batch": 64, "seq_len": "U[512,4096]", "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128,
    "block_size": 16, "work_split": "automatic balanced chunks (partition=0)", "kv_dtype": "int8/int8",
}

if __name__ == "__main__":
    main()
