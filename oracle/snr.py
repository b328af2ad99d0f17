"""Signal-to-noise ratio of an attention row -- TEST INFRASTRUCTURE.

Page "差分注意力" (aiknowledge.cn), part 二 Step 3: for a query with one true
signal position among noise positions, the ratio is the weight on the signal
position divided by the mean weight on the noise positions; differential
attention should raise it relative to plain softmax.

The signed ratio follows that definition literally.  Because a differential
row can carry negative weights, a second figure divides by the mean absolute
noise weight (a reading the page does not fix; it is reported beside the
literal one).
"""
from __future__ import annotations

import numpy as np


def snr_from_weights(a1: np.ndarray, a2: np.ndarray, lam: float, signal: int, visible: int):
    """SNRs of plain softmax (A1) and of differential attention (A1 - lam A2).

    a1, a2: float64 softmax rows; the first ``visible`` entries are the keys the
    query sees; ``signal`` is the signal position among them.
    Returns dict(plain, diff, diff_abs).
    """
    a1 = np.asarray(a1[:visible], dtype=np.float64)
    a2 = np.asarray(a2[:visible], dtype=np.float64)
    w = a1 - float(lam) * a2
    noise = np.ones(visible, dtype=bool)
    noise[signal] = False
    plain = a1[signal] / a1[noise].mean()
    diff = w[signal] / w[noise].mean()
    diff_abs = w[signal] / np.abs(w[noise]).mean()
    return {"plain": float(plain), "diff": float(diff), "diff_abs": float(diff_abs)}


def snr_closed_form(a: float, b: float, lam: float, visible: int):
    """SNRs from the signal weights alone, using that every softmax row sums to 1.

    With a = A1[signal], b = A2[signal] and n = visible - 1 noise positions, the
    noise weights of A1 sum to 1 - a and those of A1 - lam A2 to
    (1 - a) - lam (1 - b) (rows of a softmax sum to one: page "Understanding
    Differential Transformer...", 关键设计).  Hence
        plain = a n / (1 - a),  diff = (a - lam b) n / ((1 - a) - lam (1 - b)).
    """
    n = visible - 1
    plain = a * n / (1.0 - a)
    diff = (a - lam * b) * n / ((1.0 - a) - lam * (1.0 - b))
    return {"plain": float(plain), "diff": float(diff)}
