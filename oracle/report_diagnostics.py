"""Print the oracle diagnostics (pooled support at mass 0.9 over pools of
8 queries; affine-explainable fraction and orthogonal energy of the
residual) for the response-coupled and the semantic partition on reduced
synthetic workloads.  Usage: python -m oracle.report_diagnostics"""
import sys

from synth import as_f64, get_config, make_qkv, with_overrides

from .diagnostics import head_diagnostics

WORKLOADS = {
    "video AR(1), 13x45x56 reduced to 3x30x40": with_overrides(get_config(2), H=1, N=3600, frames=3, lat_h=30,
                                                              lat_w=40, G_k=48, G_q=48, M=64, rank=16, density=0.22),
    "world model Zipf, reduced to 5x30x60": with_overrides(get_config(4), H=1, N=9000, frames=5, lat_h=30, lat_w=60,
                                                          G_k=64, G_q=64, M=128, rank=32, density=0.22),
}


def main():
    print("| workload | partition | density | per-query support (median) | pooled support, 8 queries (median) "
          "| affine-explained | orthogonal energy / dense energy |")
    print("|---|---|---:|---:|---:|---:|---:|")
    for name, cfg in WORKLOADS.items():
        Q, K, V = make_qkv(cfg)
        q, k, v = as_f64(Q[0]), as_f64(K[0]), as_f64(V[0])
        for part in ("response", "semantic"):
            r = head_diagnostics(q, k, v, with_overrides(cfg, partition=part))
            print(f"| {name} | {part} | {r['density']:.3f} | {r['per_query_support_median']:.3f} | "
                  f"{r['pooled_support_median']:.3f} | {r['affine_explained']:.3f} | {r['orthogonal_energy']:.4f} |")
            sys.stdout.flush()


if __name__ == "__main__":
    main()
