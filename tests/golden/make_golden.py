"""Write the regression fixtures in this folder.  Calls only synth/ and oracle/.

The pages print no worked example for this layer, so these fixtures are not
the pages' numbers: they freeze the generator's draws (integers) and a few
oracle outputs on the tiny workload, so that an unintended change to either
shows up.  Run:  python tests/golden/make_golden.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    cfg = synth.config("varlen")
    cu = synth.cu_from_lengths(cfg.lengths)
    tab, first = oracle.chunk_table(cu, cfg.chunk)
    with open(os.path.join(HERE, "varlen_row.txt"), "w") as f:
        f.write("# varlen packed row, seed 2: lengths, cu_seqlens, chunks per sequence (chunk 64)\n")
        f.write("lengths " + " ".join(str(x) for x in cfg.lengths) + "\n")
        f.write("cu " + " ".join(str(int(x)) for x in cu) + "\n")
        f.write("chunks " + " ".join(str(int(first[i + 1] - first[i])) for i in range(len(cfg.lengths))) + "\n")
        f.write("n_chunks %d\n" % len(tab))

    cfg = synth.config("tiny")
    inp = synth.make_inputs(cfg)
    out = oracle.layer_fwd(cfg, inp)
    rng = np.random.default_rng(1234)
    with open(os.path.join(HERE, "tiny_oracle.txt"), "w") as f:
        f.write("# tiny workload (seed 0), fp64 oracle: name flat_index value\n")
        for name in ("y_conv", "o", "ht"):
            a = out[name].reshape(-1)
            for idx in sorted(rng.choice(a.size, size=12, replace=False)):
                f.write("%s %d %.17g\n" % (name, idx, a[idx]))


if __name__ == "__main__":
    main()
