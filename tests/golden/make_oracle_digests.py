"""Write tests/golden/oracle_digests.txt: SHA-256 digests of the oracle's
outputs on the tiny seeded workloads.  Calls only the oracle and the seeded
input generators.  Re-run (and say why in the commit) only when a change to
the oracle's arithmetic is justified by the pages or by a reading of them.

    python tests/golden/make_oracle_digests.py
"""
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from dequantize_reduce_transfer_amd import workloads  # noqa: E402


def digests():
    out = {}
    xs = [workloads.bits(workloads.tiny_gradient(p)) for p in range(4)]
    for fmt, name in ((oracle.E4M3, "e4m3"), (oracle.E5M2, "e5m2")):
        qs, ss = zip(*[oracle.quantize(x, fmt) for x in xs])
        out["quantize_tiny_seed0_%s_q" % name] = qs[0]
        out["quantize_tiny_seed0_%s_scales" % name] = ss[0]
        out["dequantize_tiny_seed0_%s_f32" % name] = oracle.dequantize(qs[0], ss[0], fmt)
        out["reduce_tiny_k4_%s_f32" % name] = oracle.dequant_reduce(list(qs), list(ss), fmt)
        out["reduce_tiny_k4_%s_bf16" % name] = oracle.dequant_reduce(list(qs), list(ss), fmt, True)
        rq, rs = oracle.reduce_requantize(list(qs), list(ss), fmt, fmt)
        out["reduce_requantize_tiny_k4_%s_q" % name] = rq
        out["reduce_requantize_tiny_k4_%s_scales" % name] = rs
        tq, ts = oracle.quantize_tensorwise(xs[0], fmt)
        out["quantize_tensorwise_tiny_seed0_%s_q" % name] = tq
        out["quantize_tensorwise_tiny_seed0_%s_scale" % name] = ts
    w = workloads.bits(workloads.kaiming_uniform((4, 768, 2048), seed=0))
    q, e = oracle.mx8_quantize(w)
    out["mx8_kaiming_4x768x2048_q"] = q
    out["mx8_kaiming_4x768x2048_e8m0"] = e
    q2 = q.reshape(-1, 2048)
    out["mx8_dequantize_kaiming_4x768x2048_f32"] = oracle.mx8_dequantize(q2, e)
    w2 = workloads.bits(workloads.kaiming_uniform((4, 768, 2048), seed=1))
    qb, eb = oracle.mx8_quantize(w2)
    out["mx8_reduce_kaiming_k2_f32"] = oracle.mx8_dequant_reduce([q2, qb.reshape(-1, 2048)], [e, eb])
    return {k: hashlib.sha256(v.tobytes()).hexdigest() for k, v in out.items()}


if __name__ == "__main__":
    path = os.path.join(HERE, "oracle_digests.txt")
    with open(path, "w") as f:
        f.write("# SHA-256 of oracle outputs on seeded tiny workloads; written by\n")
        f.write("# tests/golden/make_oracle_digests.py (calls only oracle/ and the input generators)\n")
        for k, v in sorted(digests().items()):
            f.write("%s %s\n" % (k, v))
    print("wrote", path)
