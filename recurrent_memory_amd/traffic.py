"""HBM traffic and matrix-core use of the EDA kernels, from rocprofv3 counters.

Two steps (the first is the program rocprofv3 profiles, once per counter):

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d FETCH_DIR -o t -- \\
        python3 REPO/recurrent_memory_amd/traffic.py run --workload train
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d WRITE_DIR -o t -- \\
        python3 REPO/recurrent_memory_amd/traffic.py run --workload train
    python3 REPO/recurrent_memory_amd/traffic.py summarize FETCH_DIR WRITE_DIR --workload train

Matrix-core use (one pass, four counters):

    rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES \\
        GRBM_GUI_ACTIVE --output-format csv -d MFMA_DIR -o t -- \\
        python3 REPO/recurrent_memory_amd/traffic.py run --workload train
    python3 REPO/recurrent_memory_amd/traffic.py summarize-mfma MFMA_DIR --workload train

`run` builds the workload's inputs, then launches a calibration kernel that
reads and writes a known number of bytes (an fp32 scale of 256 MiB, three
times), then three chunked forwards (for the decode workload: three decode
steps, state in place).  `summarize` scales each kernel's
FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what the same counter reported
for the calibration kernel and writes profiles/traffic_<kernel>_<workload>.txt,
tagged with the SHA-1 of the kernel source so that stale figures are not used.
Figures are per forward step: the state side of a step is every dispatch of
its kernels (with few heads, the segment maps, their prefix and the pass).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CALIB_BYTES = 256 << 20
NCALIB = 3
KERNELS = {"eda_bf16_factors": "eda_bf16.hip", "eda_bf16_state": "eda_bf16.hip",
           "eda_decode_kernel": "eda_decode.hip"}
# the dispatches that make up each family in one forward step
FAMILY = {"eda_bf16_factors": ("eda_bf16_factors",),
          "eda_bf16_state": ("eda_bf16_state", "eda_bf16_combine"),
          "eda_decode_kernel": ("eda_decode_kernel",)}
NSTEPS = 3


def run(workload: str) -> None:
    sys.path.insert(0, ROOT)
    import torch

    import recurrent_memory_amd as eda
    from eda_inputs import WORKLOADS, make_workload

    dev = torch.device("cuda:0")
    w = WORKLOADS[workload]
    x = make_workload(w, device=dev)
    decode = w.T == 1
    if decode:
        S = x["S0"].clone()
        o = torch.empty((w.B, w.H, w.dv), dtype=x["q"].dtype, device=dev)
    else:
        o = torch.empty((w.B, w.T, w.H, w.dv), dtype=x["q"].dtype, device=dev)
        S = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(NCALIB):
        torch.mul(src, 1.0, out=dst)   # reads and writes CALIB_BYTES each
    torch.cuda.synchronize()
    for t in range(3):
        if decode:
            eda.recurrent_step(*(x[n][t] for n in ("q", "k", "e", "v", "alpha", "beta", "gamma")), S,
                               S_out=S, o=o)
        else:
            eda.fwd_chunked(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], x["S0"],
                            out=o, S_final=S)
    torch.cuda.synchronize()
    print(f"[traffic] ran calibration and 3 {'decode steps' if decode else 'forwards'} of {workload}",
          flush=True)


def per_dispatch(directory: str, counter: str):
    """[(dispatch id, kernel name, value in KiB)] in dispatch order."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    tot, names = defaultdict(float), {}
    for row in csv.DictReader(open(files[0])):
        if row["Counter_Name"] != counter:
            continue
        d = int(row["Dispatch_Id"])
        tot[d] += float(row["Counter_Value"])
        names[d] = row["Kernel_Name"]
    return [(d, names[d], tot[d]) for d in sorted(tot)]


def summarize(fetch_dir: str, write_dir: str, workload: str, algorithmic: dict) -> None:
    out = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = per_dispatch(directory, counter)
        first_eda = next(i for i, r in enumerate(rows) if "eda_" in r[1])
        calib = rows[first_eda - NCALIB:first_eda]
        calib_kib = sum(r[2] for r in calib) / len(calib)
        scale = CALIB_BYTES / (calib_kib * 1024.0)
        for kern in KERNELS:
            vals = [r[2] for r in rows if any(n in r[1] for n in FAMILY[kern])]
            if vals:
                out.setdefault(kern, {})[counter] = (sum(vals) / NSTEPS, calib_kib, scale)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for kern, src in KERNELS.items():
        if kern not in out or len(out[kern]) != 2:
            continue
        fk, fc, fs = out[kern]["FETCH_SIZE"]
        wk, wc, wsc = out[kern]["WRITE_SIZE"]
        sha = hashlib.sha1(open(os.path.join(HERE, "csrc", src), "rb").read()).hexdigest()
        total = fk * 1024 * fs + wk * 1024 * wsc
        path = os.path.join(ROOT, "profiles", f"traffic_{kern}_{workload}.txt")
        with open(path, "w") as f:
            f.write(f"# HBM traffic per forward step of {kern} on the {workload} workload (summed over\n"
                    f"# the step's dispatches of {', '.join(FAMILY[kern])}), from rocprofv3\n"
                    "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over instances), each\n"
                    f"# scaled by the same counter on a calibration kernel that reads and writes\n"
                    f"# {CALIB_BYTES} bytes.  Commands (repo at REPO):\n"
                    "#   cd /tmp && export TMPDIR=/tmp\n"
                    "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d F -o t -- "
                    f"python3 REPO/recurrent_memory_amd/traffic.py run --workload {workload}\n"
                    "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d W -o t -- "
                    f"python3 REPO/recurrent_memory_amd/traffic.py run --workload {workload}\n"
                    f"#   python3 REPO/recurrent_memory_amd/traffic.py summarize F W --workload {workload}\n")
            f.write(f"kernel = {kern}\nworkload = {workload}\nsource = {src}\nsource_sha1 = {sha}\n")
            f.write(f"calibration_bytes = {CALIB_BYTES}\n")
            f.write(f"fetch_kib_calibration = {fc:.1f}\nfetch_scale = {fs:.4f}\nfetch_kib = {fk:.1f}\n")
            f.write(f"write_kib_calibration = {wc:.1f}\nwrite_scale = {wsc:.4f}\nwrite_kib = {wk:.1f}\n")
            f.write(f"fetch_bytes = {fk * 1024 * fs:.0f}\nwrite_bytes = {wk * 1024 * wsc:.0f}\n")
            f.write(f"bytes_per_launch = {total:.0f}\n")
            if kern in algorithmic:
                f.write(f"algorithmic_bytes = {algorithmic[kern]:.0f}\n"
                        f"traffic_over_algorithmic = {total / algorithmic[kern]:.3f}\n")
        print(f"[traffic] {path}: {total / 1e6:.1f} MB per launch")


N_XCC, N_SIMD = 8, 1024   # MI355X: 8 XCDs, 256 compute units x 4 SIMDs


def summarize_mfma(directory: str, workload: str, canonical: dict) -> None:
    """Per forward step of each chunked kernel family: the bf16 matrix operations issued
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts add and multiply operations / 512),
    the matrix-core busy fraction (SQ_VALU_MFMA_BUSY_CYCLES summed over the
    SIMDs, over the kernel's GRBM_GUI_ACTIVE cycles -- summed over the XCDs in
    the CSV -- times the SIMD count), and the issued rate against the dense
    bf16 peak over the same cycles."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    vals = defaultdict(lambda: defaultdict(list))
    per = defaultdict(dict)
    names = {}
    for row in csv.DictReader(open(files[0])):
        d = int(row["Dispatch_Id"])
        per[d][row["Counter_Name"]] = per[d].get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
        names[d] = row["Kernel_Name"]
    for d, c in per.items():
        for kern in ("eda_bf16_factors", "eda_bf16_state"):
            if any(n in names[d] for n in FAMILY[kern]):
                for k, v in c.items():
                    vals[kern][k].append(v)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for kern, c in vals.items():
        # per forward step: the sum over the step's dispatches of the family
        avg = {k: sum(v) / NSTEPS for k, v in c.items()}
        cycles = avg["GRBM_GUI_ACTIVE"] / N_XCC
        issued = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_SIMD)
        # dense bf16 peak: 1024 flop per SIMD per cycle (2.5 PFLOP/s at 2.4 GHz over 1024 SIMDs;
        # a 16x16x32 bf16 instruction is 16384 flop in 16 busy cycles)
        rate = issued / (cycles * N_SIMD * 1024.0)
        sha = hashlib.sha1(open(os.path.join(HERE, "csrc", KERNELS[kern]), "rb").read()).hexdigest()
        path = os.path.join(ROOT, "profiles", f"mfma_{kern}_{workload}.txt")
        with open(path, "w") as f:
            f.write(f"# Matrix-core use per forward step of {kern} on the {workload} workload (summed\n"
                    f"# over the step's dispatches of {', '.join(FAMILY[kern])}), from rocprofv3 counters.\n"
                    "# Commands (repo at REPO):\n"
                    "#   cd /tmp && export TMPDIR=/tmp\n"
                    "#   rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES "
                    f"GRBM_GUI_ACTIVE --output-format csv -d M -o t -- python3 REPO/recurrent_memory_amd/traffic.py "
                    f"run --workload {workload}\n"
                    f"#   python3 REPO/recurrent_memory_amd/traffic.py summarize-mfma M --workload {workload}\n")
            f.write(f"kernel = {kern}\nworkload = {workload}\nsource = {KERNELS[kern]}\nsource_sha1 = {sha}\n")
            f.write(f"dispatches = {len(c['GRBM_GUI_ACTIVE'])} over {NSTEPS} forward steps\n")
            for k in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES",
                      "GRBM_GUI_ACTIVE"):
                f.write(f"{k} = {avg[k]:.0f}\n")
            f.write(f"gpu_active_cycles_per_xcd = {cycles:.0f}\n")
            f.write(f"issued_bf16_flop = {issued:.0f}\n")
            if kern in canonical:
                f.write(f"canonical_flop = {canonical[kern]:.0f}\n"
                        f"issued_over_canonical = {issued / canonical[kern]:.3f}\n")
            f.write(f"mfma_busy_fraction = {busy:.4f}\n")
            f.write(f"issued_rate_over_bf16_peak = {rate:.4f}\n")
        print(f"[mfma] {path}: busy {100 * busy:.1f} %, issued {issued / 1e9:.2f} GFLOP")


def canonical_flop(workload: str, chunk: int = 0) -> dict:
    """The chunk formulation's multiply-adds x 2 per launch (counted once), at
    `chunk` tokens per chunk (0: the library default, which `run` uses)."""
    sys.path.insert(0, ROOT)
    from eda_inputs import WORKLOADS
    w = WORKLOADS[workload]
    if chunk == 0:
        import recurrent_memory_amd as eda
        chunk = eda.DEFAULT_CHUNK
    C, L, d = chunk, 2 * chunk, w.dk
    n = w.B * w.H * ((w.T + C - 1) // C)
    return {"eda_bf16_factors": 2.0 * n * (L * L * d + L ** 3 / 6.0 + L * L * d + C * L * d),
            "eda_bf16_state": 2.0 * n * (L * d * d + L * C * d + C * d * d + C * L * d + L * d * d)}


def algorithmic_bytes(workload: str) -> dict:
    sys.path.insert(0, ROOT)
    from eda_inputs import WORKLOADS
    w = WORKLOADS[workload]
    es = 2 if w.dtype == "bf16" else 4
    n = w.B * w.T * w.H
    state_io = (2 if w.s0_std > 0 else 1) * w.B * w.H * w.dk * w.dv * 4
    return {"eda_bf16_factors": n * (3 * w.dk * es + w.dk * 4 + 8),
            "eda_bf16_state": n * (2 * w.dv * es) + state_io,
            # decode: the state read and written, one token's q, k, e, v, alpha,
            # beta, gamma in and o out per (sequence, head)
            "eda_decode_kernel": w.B * w.H * (2 * w.dk * w.dv * 4 + (3 * w.dk + 2 * w.dv) * es + w.dk * 4 + 8)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="train")
    sm = sub.add_parser("summarize")
    sm.add_argument("fetch_dir")
    sm.add_argument("write_dir")
    sm.add_argument("--workload", default="train")
    mf = sub.add_parser("summarize-mfma")
    mf.add_argument("mfma_dir")
    mf.add_argument("--workload", default="train")
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.workload)
    elif a.cmd == "summarize-mfma":
        summarize_mfma(a.mfma_dir, a.workload, canonical_flop(a.workload))
    else:
        summarize(a.fetch_dir, a.write_dir, a.workload, algorithmic_bytes(a.workload))
    return 0


if __name__ == "__main__":
    sys.exit(main())
