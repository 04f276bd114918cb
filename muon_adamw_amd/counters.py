"""HBM traffic per kernel launch from rocprofv3 counter passes.

rocprofv3 reports FETCH_SIZE and WRITE_SIZE in KiB per dispatch, summed over
the L2 channels of the chip. Their scale is calibrated in the same runs on a
plain device copy of known size (1 GiB read + 1 GiB written, torch's copy
kernel): factor = true KiB / counted KiB for each counter. The summary keeps
the per-launch averages of every library kernel, the two factors and a hash of
the kernel sources, so a reader can tell whether the numbers still describe
the code (bench.py reports them only while the hash matches).

Matrix-core work comes from an optional third pass with an MFMA-op counter
(SQ_INSTS_VALU_MFMA_MOPS_BF16 by default), calibrated the same way on the
MFMA-only ceiling loop that bench.py runs (CEILING_BLOCKS workgroups of four
waves, CEILING_ITERS rounds of eight 32x32x16 bf16 multiplies: a known number
of flops), so that no counter unit has to be assumed. The summary then gives
the flops the matrix cores executed per launch, to hold against the
algorithmic count (the gap is padding and the full diagonal tiles).

Usage:
  python -m muon_adamw_amd.counters --fetch FETCH.csv --write WRITE.csv [--mfma MFMA.csv] \
      --workload gpt_12L_d768 --command "..." --out profiles/counters_gpt_12L_d768.json
"""
import argparse
import collections
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
COPY_BYTES = 1 << 30
# the MFMA-only ceiling launch bench.py times: its flops are known exactly
CEILING_BLOCKS = 1024
CEILING_ITERS = 1000
CEILING_FLOPS = CEILING_BLOCKS * 4 * CEILING_ITERS * 8 * (32 * 32 * 16 * 2)
MFMA_COUNTER = "SQ_INSTS_VALU_MFMA_MOPS_BF16"

# kernel symbol -> the name the library's per-kernel timing uses
_NAMES = [
    (r"ns_persistent_kernel", "ns_persistent_bf16"), (r"ns_mfma_kernel<0>", "ns_gram_bf16"), (r"ns_mfma_kernel<1>", "ns_square_bf16"),
    (r"ns_mfma_kernel<2>", "ns_apply_bf16"), (r"ns_f32_kernel<0>", "ns_gram_f32"),
    (r"ns_f32_kernel<1>", "ns_square_f32"), (r"ns_f32_kernel<2>", "ns_apply_f32"),
    (r"momentum_kernel", "momentum"), (r"norm_finalize_kernel", "norm_finalize"),
    (r"apply_kernel", "apply_update"), (r"adamw_kernel", "adamw"),
    (r"canon_rowsum_kernel", "rowsum"), (r"canon_colsum_kernel", "colsum"),
    (r"finalize_normuon_kernel", "finalize_normuon"), (r"finalize_muon_plus_kernel", "finalize_muon_plus"),
    (r"grad_sumsq_kernel", "grad_sumsq"), (r"grad_norm_finalize_kernel", "grad_norm_finalize"),
    (r"mfma_ceiling_kernel", "mfma_ceiling"),
]


def source_hash() -> str:
    """sha256 over the kernel sources (every file of csrc/, sorted by name)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def _kernel_name(symbol: str):
    for pat, name in _NAMES:
        if re.search(pat, symbol):
            return name
    if "copy" in symbol.lower() or "Copy" in symbol:
        return "copy"
    return None


def _load(path, counter):
    """Per-dispatch values of one counter, grouped by kernel name."""
    per = collections.defaultdict(list)
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] != counter:
            continue
        name = _kernel_name(row["Kernel_Name"])
        if name is None:
            continue
        per[name].append((int(row.get("Grid_Size", 0) or 0), float(row["Counter_Value"])))
    return per


def _copy_kib(vals, what="copy kernel"):
    """Counted value of the calibration launch: the dispatches within a factor
    of two of the largest (the 1 GiB copies, or the full-length ceiling loop;
    other launches of the run, such as input staging or the ceiling's short
    warm-up, are far smaller), averaged."""
    if not vals:
        raise ValueError(f"no {what} dispatches in the counter file")
    top = max(v for _, v in vals)
    big = [v for _, v in vals if v >= 0.5 * top]
    return sum(big) / len(big)


def summarize(fetch_csv, write_csv, workload, command, mfma_csv=None, mfma_counter=MFMA_COUNTER):
    fe = _load(fetch_csv, "FETCH_SIZE")
    wr = _load(write_csv, "WRITE_SIZE")
    true_kib = COPY_BYTES / 1024.0
    ff = true_kib / _copy_kib(fe.pop("copy", []))
    wf = true_kib / _copy_kib(wr.pop("copy", []))
    kernels = {}
    for name in sorted(set(fe) | set(wr)):
        f = [v for _, v in fe.get(name, [])]
        w = [v for _, v in wr.get(name, [])]
        if not f or not w:
            continue
        fk, wk = sum(f) / len(f), sum(w) / len(w)
        kernels[name] = {"dispatches": len(f), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                         "hbm_bytes_per_launch": round((fk * ff + wk * wf) * 1024.0)}
    out = {"workload": workload, "command": command, "fetch_factor": round(ff, 4),
           "write_factor": round(wf, 4), "source_sha256": source_hash(), "kernels": kernels}
    if mfma_csv:
        mf = _load(mfma_csv, mfma_counter)
        mfac = CEILING_FLOPS / _copy_kib(mf.pop("mfma_ceiling", []), "MFMA ceiling loop")
        for name, vals in sorted(mf.items()):
            v = [x for _, x in vals]
            k = kernels.setdefault(name, {"dispatches": len(v)})
            k["mfma_flops_per_launch"] = round(sum(v) / len(v) * mfac)
        out.update(mfma_counter=mfma_counter, mfma_factor=mfac)
    return out


def traffic_for(summary_path, kernel):
    """HBM bytes per launch of `kernel` from a committed summary, or None when
    there is none or the kernel sources changed since it was taken."""
    if not os.path.exists(summary_path):
        return None
    s = json.load(open(summary_path))
    if s.get("source_sha256") != source_hash():
        return None
    return s.get("kernels", {}).get(kernel, {}).get("hbm_bytes_per_launch")


def flops_for(summary_path, kernel):
    """Matrix-core flops per launch of `kernel` from a committed summary, or
    None (no summary, no MFMA pass, or kernel sources changed since)."""
    if not os.path.exists(summary_path):
        return None
    s = json.load(open(summary_path))
    if s.get("source_sha256") != source_hash():
        return None
    return s.get("kernels", {}).get(kernel, {}).get("mfma_flops_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--mfma", default=None, help="counter CSV of an MFMA-op counter pass")
    ap.add_argument("--mfma-counter", default=MFMA_COUNTER)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()
    s = summarize(a.fetch, a.write, a.workload, a.command, a.mfma, a.mfma_counter)
    with open(a.out, "w") as f:
        json.dump(s, f, indent=1)
        f.write("\n")
    print(json.dumps(s, indent=1))


if __name__ == "__main__":
    main()
