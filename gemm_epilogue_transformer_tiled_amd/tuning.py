"""Offline tile-config search and the cache that plan creation consults.

``gemm_epilogue_create`` picks a kernel instance by a rule (the largest tile that still
gives at least 256 workgroups, one per compute unit).  This module replaces the rule by
measurement where a shape is worth it: it times every admissible instance on the actual
problem and records the fastest under the problem's signature in a JSON cache; plans built
through ``runner.prepare(..., cache=...)`` then request that instance through the
descriptor's ``tile`` field.

Sources (pages as titled): the TileLang tutorial's schedule-exploration paragraph defines an
autotuning search space over tile sizes (and K block, pipeline depth, threads), filters out
configurations beyond the shared-memory budget, and benchmarks, validates and caches the
candidates; the cuDNN Graph API tutorial's engine-autotuning paragraph times every candidate
plan instead of trusting the heuristic and keeps the fastest index for reuse.

Here the search space is the compiled instances (tile shape; the K step, pipeline depth and
wave count are fixed per instance), the budget filter is the 160 KiB of LDS per compute unit,
and "validate" is the caller's business (the tests check a tuned plan against the oracle).
Argument marshalling and timing only: every candidate runs the HIP kernels.
"""
from __future__ import annotations

import dataclasses
import json
import os
from typing import Callable, Dict, List, Optional

from . import GE_OK, GE_OP_PAIRWISE_ACT_MUL, GE_TILE_COUNT, ge_desc_t, gemm_epilogue_tile_info, gemm_epilogue_validate

LDS_PER_CU = 160 * 1024          # MI355X (gfx950): LDS bytes per compute unit


def admissible_tiles(desc: ge_desc_t, lds_budget: int = LDS_PER_CU) -> List[int]:
    """Instances whose pairwise-ness matches the descriptor's chain, that the library accepts
    for it (the two-wave instances cover forward chains on bf16 operands, B [K][N], K a
    multiple of 64) and whose workgroup LDS fits the budget, in id order."""
    pair = any(desc.ops[i].kind == GE_OP_PAIRWISE_ACT_MUL for i in range(desc.n_ops))
    out = []
    for t in range(GE_TILE_COUNT):
        info = gemm_epilogue_tile_info(t)
        if bool(info.pairwise) != pair or info.lds_bytes > lds_budget:
            continue
        d = ge_desc_t.from_buffer_copy(desc)
        d.tile = t + 1
        if gemm_epilogue_validate(d) == GE_OK:
            out.append(t)
    return out


def signature(desc: ge_desc_t) -> str:
    """Cache key: shape, operand and output types, B layout and the epilogue chain (op kinds
    and activations)."""
    ops = ",".join(f"{desc.ops[i].kind}:{desc.ops[i].act}" for i in range(desc.n_ops))
    return (f"b{desc.batch}_m{desc.M}_n{desc.N}_k{desc.K}_a{desc.a_type}_b{desc.b_type}_y{desc.y_type}"
            f"_l{desc.b_layout}_ops[{ops}]")


@dataclasses.dataclass
class TileCache:
    """JSON file: {signature: {"tile": id, "ms": {id: ms per launch}}}."""

    path: str
    entries: Dict[str, dict] = dataclasses.field(default_factory=dict)

    @classmethod
    def load(cls, path: str) -> "TileCache":
        entries = {}
        if os.path.exists(path):
            with open(path) as f:
                entries = json.load(f)
        return cls(path, entries)

    def lookup(self, desc: ge_desc_t) -> Optional[int]:
        e = self.entries.get(signature(desc))
        return None if e is None else int(e["tile"])

    def record(self, desc: ge_desc_t, timings: Dict[int, float]) -> int:
        best = min(timings, key=timings.get)
        self.entries[signature(desc)] = {"tile": best, "ms": {str(k): round(v, 6) for k, v in timings.items()}}
        return best

    def save(self) -> None:
        tmp = self.path + ".tmp"
        with open(tmp, "w") as f:
            json.dump(self.entries, f, indent=1, sort_keys=True)
        os.replace(tmp, self.path)


def sweep(desc: ge_desc_t, make_run: Callable[[int], Callable[[], None]], steps: int = 20, warmup: int = 5,
          lds_budget: int = LDS_PER_CU) -> Dict[int, float]:
    """Times every admissible instance: ``make_run(tile)`` returns a callable that enqueues one
    launch of a plan built with that tile on the current stream.  Returns {tile: ms per launch}
    over `steps` back-to-back launches bracketed by HIP events (device synchronised)."""
    import torch

    stream = torch.cuda.current_stream()
    out: Dict[int, float] = {}
    for t in admissible_tiles(desc, lds_budget):
        run = make_run(t)
        for _ in range(warmup):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        out[t] = e0.elapsed_time(e1) / steps
    return out
