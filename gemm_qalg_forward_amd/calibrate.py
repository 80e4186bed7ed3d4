"""Tile calibration of the row-typed forward on the current GPU.

Times qalg_forward on one shape with every output-tile height the persistent
forward offers (QALG_FLAG_TILE_M64 / M128 / M256), the register-staged tiled
kernel (QALG_FLAG_FORCE_TILED), both few-rows schedules (section 5.3's
two-stage schedule, QALG_FLAG_TWO_STAGE, and the masked tile over all rows,
QALG_FLAG_MASKED) and the default choice, on seeded synthetic bf16 operands,
and prints the times.  Section 5.3 and appendix F of arXiv 2609.32814
calibrate tiles and both schedules per shape the same way (a short sweep,
then the chosen configuration).

    python -m gemm_qalg_forward_amd.calibrate --M 2048 --K 4096 --N 12288 --q 32
"""
from __future__ import annotations

import argparse
import json

import gemm_qalg_forward_amd as Q

CANDIDATES = [
    ("default", 0),
    ("persistent_m64", Q.QALG_FLAG_TILE_M64),
    ("persistent_m128", Q.QALG_FLAG_TILE_M128),
    ("persistent_m256", Q.QALG_FLAG_TILE_M256),
    ("tiled", Q.QALG_FLAG_FORCE_TILED),
    ("two_stage", Q.QALG_FLAG_TWO_STAGE),
    ("masked", Q.QALG_FLAG_MASKED),
]


def sweep(M: int, K: int, N: int, q: int, law: int = 0, reps: int = 20, warmup: int = 3, seed: int = 1,
          rounds: int = 3, stream=None) -> dict:
    """{candidate: median ms per launch over `rounds` interleaved rounds} for the candidates this
    shape accepts (others are left out).  The rounds alternate the candidates so that the GPU's
    power state drifts over all of them alike."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    X = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    W = (torch.randn(K, N, device="cuda", generator=g) * K ** -0.5).to(torch.bfloat16)
    tau = (torch.arange(M, device="cuda") % q).to(torch.int32)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ws = Q.workspace(q, M, two_stage_N=N)   # room for the two-stage schedule's diagonal maps
    Q.qalg_build_index(tau, q, ws=ws, stream=stream)
    runs = {}
    for name, flag in CANDIDATES:
        if law and flag in (Q.QALG_FLAG_FORCE_TILED, Q.QALG_FLAG_TWO_STAGE, Q.QALG_FLAG_MASKED):
            continue
        fl = flag | law | Q.QALG_FLAG_INDEX_READY

        def run(fl=fl):
            Q.qalg_forward(X, W, tau, q, Y=Y, ws=ws, flags=fl, stream=stream)

        try:
            run()
        except Q.QalgError:
            continue  # the shape cannot use this candidate
        runs[name] = run
    times = {name: [] for name in runs}
    for _ in range(rounds):
        for name, run in runs.items():
            for _ in range(warmup):
                run()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                run()
            b.record()
            torch.cuda.synchronize()
            times[name].append(a.elapsed_time(b) / reps)
    return {name: sorted(t)[len(t) // 2] for name, t in times.items()}


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--M", type=int, required=True)
    ap.add_argument("--K", type=int, required=True)
    ap.add_argument("--N", type=int, required=True)
    ap.add_argument("--q", type=int, required=True)
    ap.add_argument("--tensor-law", action="store_true", help="the recursive law Q_2^(x)L (q = 2^L)")
    ap.add_argument("--reps", type=int, default=20)
    a = ap.parse_args()
    law = Q.QALG_FLAG_LAW_TENSOR if a.tensor_law else 0
    res = sweep(a.M, a.K, a.N, a.q, law, a.reps)
    rho = (2 * a.q - 1) / a.q ** 2 if not law else 0.75 ** (a.q.bit_length() - 1)
    flop = 2.0 * rho * a.M * a.K * a.N
    print(json.dumps({k: {"ms": round(v, 4), "algebra_tflops": round(flop / (v * 1e-3) / 1e12, 1)}
                      for k, v in res.items()}))


if __name__ == "__main__":
    main()
