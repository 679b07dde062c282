"""GPU parity on a seeded sweep of random shapes: format pair, head size, KV and
query heads, batch and length mix (empty, one-token and page-edge lengths among
them), scale granularity, query tokens per sequence, work split, the cache
written token by token or converted from bf16 pages, and the call's output type.
Each case: the cache codes bit-exact against the oracle, and the attention
output within the gate of its output type (f32: 4e-3 absolute; bf16: that or
half a bf16 ulp of the oracle's value plus 1e-4)."""

import numpy as np
import pytest
import torch

from tests.kvq_harness import (assert_codes_equal, build_library_cache, build_oracle_cache, gate_errors,
                               library_decode, log, oracle_decode)
from workloads import WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu

PAIRS = [(k, v) for k in ("bf16", "int8", "e4m3", "e5m2") for v in ("bf16", "int8", "e4m3", "e5m2")]
PAIRS += [("int4", "int4"), ("int4h", "int4")]
N_CASES = 160


def _case(i):
    rng = np.random.default_rng(1000 + i)
    kd, vd = PAIRS[int(rng.integers(len(PAIRS)))]
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8]))
    B = int(rng.integers(1, 13))
    lens = rng.integers(0, 700, size=B)
    edge = np.array([0, 1, 15, 16, 17, 32, 33])
    pick = rng.random(B) < 0.3
    lens[pick] = rng.choice(edge, size=int(pick.sum()))
    if lens.max() == 0:
        lens[0] = 5                                   # at least one sequence with tokens
    n_q = 1 if rng.random() < 0.6 else int(rng.integers(2, 21))
    partition = int(rng.choice([0, 0, 16, 64, 512]))
    int4 = kd in ("int4", "int4h")
    gran = "per_token_head" if int4 else ("per_kv_head" if rng.random() < 0.3 else "per_tensor")
    mode = lambda dt: "row" if int4 else ("one" if dt == "bf16" or (dt == "e5m2" and rng.random() < 0.5) else "absmax")
    w = WORKLOADS["tiny_int8"].with_(
        name=f"sweep{i}", seed=2000 + i, B=B, Hq=g * Hkv, Hkv=Hkv, D=D, k_dtype=kd, v_dtype=vd,
        lens=("fixed", tuple(int(x) for x in lens)), n_q=n_q, new_tokens=0, partition=partition,
        k_gran="per_tensor" if kd == "bf16" else gran, v_gran="per_tensor" if vd == "bf16" else gran,
        k_scale_mode=mode(kd), v_scale_mode=mode(vd),
        calib="none" if int4 else "all", from_bf16_cache=bool(rng.random() < 0.2))
    out_dtype = "bf16" if rng.random() < 0.3 else "f32"
    return w, out_dtype


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    w, out_dtype = _case(i)
    log(f"[sweep {i}] {w.k_dtype}/{w.v_dtype} D={w.D} Hq={w.Hq} Hkv={w.Hkv} B={w.B} n_q={w.n_q} "
        f"partition={w.partition} gran={w.k_gran} convert={w.from_bf16_cache} out={out_dtype} lens={w.lens[1]}")
    inp = make_decode_inputs(w)
    r = build_library_cache(w, inp)
    o = build_oracle_cache(w, inp)
    assert int(r.err.item()) == 0
    assert_codes_equal(r, o, inp)
    out = library_decode(r, inp, partition=w.partition, out_dtype=out_dtype)
    torch.cuda.synchronize()
    mx, nbad = gate_errors(out, oracle_decode(o, inp), out_dtype)
    log(f"[sweep {i}] max|err| = {mx:.3e}")
    assert nbad == 0
