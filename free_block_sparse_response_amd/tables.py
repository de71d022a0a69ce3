"""Ablation tables of the SparsePR paper on synthetic inputs, run through the library.

Rows mirror the paper's Table 2 (partition construction with repair disabled, and the
partition-repair interaction), Table 4 (probe selection and correction family) and
Table D.2(a) (probe count at fixed lambda), plus a ridge-lambda sweep and an output-truncation
sweep (the residual fit restricted to the probe residuals' leading directions). Each entry is the
mean / p99 rel-L2 error ||O_i - O_i^dense|| / (||O_i^dense|| + 1e-8) over unprobed rows,
with the dense output from the library's own dense kernel on the same inputs.

Within a panel every configuration is evaluated on one shared set of rows: the rows that
none of the panel's probe sets contains. The Table 2 panel fixes the probe indices and
weights of the full method for every partition (the paper's repair comparisons fix them).

    python -m free_block_sparse_response_amd.tables --config c2 [--json out.json]
"""
from __future__ import annotations

import argparse
import json
import sys
import time

import torch

from . import configs, synth
from .call import SparsePR, config_from_workload

PARTITIONS = {"semantic": 1, "key-response K/V": 2, "response-coupled": 0}
SELECTORS = {"random": 1, "uniform spatiotemporal": 2, "query-group stratified": 0}


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


class Bench:
    def __init__(self, w, dev):
        self.w, self.dev = w, dev
        self.N, self.d, self.BH = configs.seq_len(w), w["head_dim"], w["batch"] * w["heads"]
        q64, k64, v64 = synth.make_inputs(w)
        self.q, self.k, self.v = (synth.cast_to_dtype(x, w["dtype"])[0].reshape(w["batch"], w["heads"], self.N,
                                                                                   self.d).to(dev)
                                  for x in (q64, k64, v64))
        sp = SparsePR(config_from_workload(w), device=dev)
        dense = torch.empty_like(self.q)
        sp.dense(self.q, self.k, self.v, dense)
        torch.cuda.synchronize()
        sp.close()
        self.ref = dense.reshape(self.BH, self.N, self.d).float()
        self.ref_norm = self.ref.norm(dim=-1)

    def run(self, probes=None, weights=None, **over):
        """One call with config overrides; probes/weights replace the plan's probe rows."""
        sp = SparsePR(config_from_workload(self.w, **over), device=self.dev)
        sp.plan(self.q, self.k)
        if probes is not None:
            sp.set_probes(probes, weights)
        sp.attend(self.q, self.k, self.v)
        sp.fit_residual()
        sp.apply()
        torch.cuda.synchronize()
        info = sp.info()
        density = sum(i["executed_pairs"] for i in info) / (len(info) * float(self.N) ** 2)
        rows_err = ((sp.out.reshape(self.BH, self.N, self.d).float() - self.ref).norm(dim=-1)
                    / (self.ref_norm + 1e-8))
        res = dict(err=rows_err, probes=sp.export("PROBES").long(), weights=sp.export("PROBE_WEIGHTS").clone(),
                   density=density)
        sp.close()
        return res

    def unprobed(self, runs):
        mask = torch.ones((self.BH, self.N), dtype=torch.bool, device=self.dev)
        for r in runs:
            mask.scatter_(1, r["probes"], False)
        return mask


def _stats(err, mask):
    e = err[mask].double()
    return float(e.mean()), float(torch.quantile(e.float(), 0.99))


def _panel(b, name, runs):
    mask = b.unprobed(runs.values())
    rows = []
    for label, r in runs.items():
        mean, p99 = _stats(r["err"], mask)
        rows.append(dict(setting=label, mean=round(mean, 5), p99=round(p99, 5), density=round(r["density"], 5)))
    _log(f"{name}: {int(mask.sum())} shared unprobed rows")
    return dict(panel=name, rows=rows, eval_rows=int(mask.sum()))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--config", default="c2", choices=sorted(configs.CONFIGS))
    ap.add_argument("--table4-probes", type=int, default=64, help="M of the Table 4 / D.2 panels (paper: 64)")
    ap.add_argument("--table4-lambda", type=float, default=1.0, help="lambda of the Table 4 / D.2 panels (paper: 1)")
    ap.add_argument("--probe-counts", default="16,32,64,128", help="M values of the Table D.2(a) panel")
    ap.add_argument("--lambdas", default="1e-3,1e-1,1,10,100", help="lambda values of the ridge sweep")
    ap.add_argument("--output-ranks", default="1,4,16,64,0",
                    help="output truncation ranks of the residual fit (0: none, the method)")
    ap.add_argument("--json", default=None, help="also write the panels to this file")
    args = ap.parse_args(argv)

    w = configs.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    b = Bench(w, dev)
    _log(f"inputs {args.config}: B*H={b.BH} N={b.N} d={b.d} ({time.perf_counter() - t0:.1f} s)")
    panels = []

    # Table 2: partitions with repair disabled, and semantic + repair, all with the probe rows
    # and weights of the full method
    full = b.run()
    fixed = dict(probes=full["probes"].int().contiguous(), weights=full["weights"].contiguous())
    t2 = {f"{k} partition, repair disabled": b.run(partition=v, correction=2, **fixed) for k, v in PARTITIONS.items()}
    t2["semantic partition + probe repair"] = b.run(partition=1, correction=0, **fixed)
    t2["SparsePR (response-coupled + probe repair)"] = full
    p2 = _panel(b, f"Table 2 (M={w['n_probes']}, lambda={w['ridge_lambda']})", t2)
    base = p2["rows"][0]["mean"]
    for r in p2["rows"]:
        r["reduction_vs_semantic_no_repair"] = round((base - r["mean"]) / base, 4) if base > 0 else None
    panels.append(p2)

    # Table 4: probe selection (full weighted ridge) and the mean-only correction
    m4, l4 = args.table4_probes, args.table4_lambda
    t4 = {f"{k} probes": b.run(n_probes=m4, ridge_lambda=l4, probe_selector=v) for k, v in SELECTORS.items()}
    t4["mean-only correction (stratified probes)"] = b.run(n_probes=m4, ridge_lambda=l4, correction=1)
    panels.append(_panel(b, f"Table 4 (M={m4}, lambda={l4})", t4))

    # Table D.2(a): probe count at fixed lambda
    td = {f"M={m}": b.run(n_probes=m, ridge_lambda=l4) for m in (int(x) for x in args.probe_counts.split(","))}
    panels.append(_panel(b, f"Table D.2(a) (lambda={l4})", td))

    # ridge lambda at the workload's probe count
    tl = {f"lambda={lam:g}": b.run(ridge_lambda=lam) for lam in (float(x) for x in args.lambdas.split(","))}
    panels.append(_panel(b, f"lambda sweep (M={w['n_probes']})", tl))

    # output truncation of the residual fit at the workload's M and lambda ([D.2] "no output
    # truncation" is the method's setting, rank 0 here)
    tr = {(f"rank {r}" if r else "no truncation"): b.run(output_rank=r)
          for r in (int(x) for x in args.output_ranks.split(","))}
    panels.append(_panel(b, f"output truncation (M={w['n_probes']}, lambda={w['ridge_lambda']})", tr))

    for p in panels:
        print(f"\n{p['panel']} - mean / p99 unprobed rel-L2 over {p['eval_rows']} shared rows")
        for r in p["rows"]:
            extra = f"  (-{100 * r['reduction_vs_semantic_no_repair']:.1f}%)" if "reduction_vs_semantic_no_repair" in r else ""
            print(f"  {r['setting']:<48} {r['mean']:.4f} / {r['p99']:.4f}  density {r['density']:.4f}{extra}")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(dict(config=args.config, panels=panels), f, indent=1)


if __name__ == "__main__":
    main()
