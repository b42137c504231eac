"""Writes closed_forms.json: hand-derived attention-residual cases whose exact
answer follows from the definition by pen and paper.

The pages print no worked numeric example, so these fixtures come from the
mathematics alone.  This script uses only Python's ``math`` and ``fractions``:
it calls neither the oracle nor the GPU library.

Definition (vllm-ascend PR #14840, "Implementation walkthrough"; vLLM PR #54261
digest, kernel snippet under "Key source snippets"): per token the sources are
the valid bank rows followed by cur (= prefix, or RNE_bf16(prefix + delta));
logit_j = sum_h rms_w[h] res_w[h] x_j[h] / sqrt(mean(x_j^2) + eps); p =
softmax(logits); y = sum_j p_j x_j (raw rows); optional out = y /
sqrt(mean(y^2) + oeps) * w_o.

With rms_w = res_w = 1 and eps = 0, a row whose entries all have magnitude c
normalises to its sign pattern, so its logit is (#positive - #negative)
entries: that is how the logits below are engineered.
"""
import json
import math
import os
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def softmax(ls):
    m = max(ls)
    e = [math.exp(l - m) for l in ls]
    z = sum(e)
    return [v / z for v in e]


def mix(p, rows):
    H = len(rows[0])
    return [math.fsum(p[j] * rows[j][h] for j in range(len(rows))) for h in range(H)]


def onorm(y, w, oeps):
    r = math.sqrt(math.fsum(v * v for v in y) / len(y) + oeps)
    return [y[h] / r * w[h] for h in range(len(y))]


def case(name, derivation, bank, prefix, delta, res_w, rms_w, onw, eps, oeps, widx,
         probs, out, cap=None):
    return dict(name=name, derivation=derivation, H=len(prefix), nb=len(bank),
                cap=cap if cap is not None else max(len(bank), widx + 1, 1),
                bank=bank, prefix=prefix, delta=delta, res_w=res_w, rms_w=rms_w,
                onw=onw, eps=eps, oeps=oeps, widx=widx, probs=probs, out=out)


def main():
    ones = [1.0] * 8
    cases = []

    # 1. Two sources, logits 8 and 2: p0 = sigmoid(6).
    x0 = [1.0] * 8
    x1 = [2.0] * 5 + [-2.0] * 3
    p0 = 1.0 / (1.0 + math.exp(-6.0))
    p = [p0, 1.0 - p0]
    y = mix(p, [x0, x1])
    cases.append(case(
        "two_sources_sigmoid",
        "x0 = 1 (all 8), logit 8; cur = (2 x5, -2 x3), normalised to signs, logit 2; "
        "p0 = 1/(1+e^-6); y = p0*x0 + (1-p0)*cur, raw rows",
        [x0], x1, None, ones, ones, None, 0.0, 0.0, -1, p, y))

    # 2. The same with an output norm of weight (1,2,1,2,...) and oeps = 0.
    w = [1.0, 2.0] * 4
    cases.append(case(
        "two_sources_sigmoid_onorm",
        "case 1 followed by out = y / sqrt(mean(y^2)) * w, w = (1,2,1,2,...)",
        [x0], x1, None, ones, ones, w, 0.0, 0.0, -1, p, onorm(y, w, 0.0)))

    # 3. Three sources with logits 4, 0, -4.
    a = [1.0] * 6 + [-1.0] * 2
    b = [3.0] * 4 + [-3.0] * 4
    c = [0.5] * 2 + [-0.5] * 6
    p3 = softmax([4.0, 0.0, -4.0])
    cases.append(case(
        "three_sources_softmax",
        "logits 4 (6 positive of 8), 0 (4 of 8), -4 (2 of 8); p = softmax(4,0,-4); "
        "y = sum p_j x_j over raw rows (cur last)",
        [a, b], c, None, ones, ones, None, 0.0, 0.0, -1, p3, mix(p3, [a, b, c])))

    # 4. Zero scoring weight: every logit is 0, so y is the plain mean of the
    #    sources; prefix + delta is exact in bf16 here, and cur is written to
    #    slot 1 (a slot that is also a source: its old value is mixed).
    s0 = [1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0]
    s1 = [-8.0, 0.5, 0.25, 16.0, -3.0, 1.5, 2.0, -0.75]
    pre = [1.0, 1.0, -2.0, 0.5, 4.0, 8.0, -1.0, 0.0]
    dl = [0.5, -3.0, 2.0, 0.25, 4.0, -8.0, 1.0, 3.0]
    cur = [pre[h] + dl[h] for h in range(8)]
    mean = [float((Fraction(s0[h]) + Fraction(s1[h]) + Fraction(cur[h])) / 3) for h in range(8)]
    cases.append(case(
        "zero_score_weight_mean",
        "res_w = 0 makes every logit 0, p = 1/3 each; y = (s0 + s1 + cur)/3 with "
        "cur = prefix + delta (exact in bf16); cur also lands in slot 1",
        [s0, s1], pre, dl, [0.0] * 8, ones, None, 1e-6, 0.0, 1,
        [1.0 / 3.0] * 3, mean, cap=3))

    # 5. No blocks: the output is the output-normalised current residual.
    cu = [1.0, -1.0] * 4
    wo = [0.5, 2.0, 4.0, -1.0, 1.0, 0.25, 3.0, 1.0]
    cases.append(case(
        "no_blocks_output_norm",
        "nb = 0, p = (1); cur = (1,-1,...), mean square 1, oeps = 0, so out = cur * w_o",
        [], cu, None, ones, ones, wo, 1e-6, 0.0, -1, [1.0], [cu[h] * wo[h] for h in range(8)]))

    with open(os.path.join(HERE, "closed_forms.json"), "w") as f:
        json.dump({"source": "hand-derived closed forms (no printed example exists on the pages)",
                   "cases": cases}, f, indent=1)


if __name__ == "__main__":
    main()
