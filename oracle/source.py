"""Host-side fp64 view of seeded decode inputs, for the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring). Converts the input tensors
to fp64 numpy arrays (an exact widening of bf16 / fp16 / fp32) and fetches raw
K/V rows on demand, so full-size caches never have to be widened whole.
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(t):
    return None if t is None else t.detach().to("cpu").double().numpy()


class HostSource:
    """Inputs of one decode step as the oracle reads them.

    ``inputs`` maps names (q, K, V, Kg, Vg, Kmg, P, Kp) to tensors on any
    device. Small arrays are widened once; K and V rows are gathered per call.
    """

    def __init__(self, inputs: dict):
        self._K = inputs["K"]
        self._V = inputs["V"]
        q = _f64(inputs["q"])
        # [B][T][Hq][d] (T adjacent query tokens) -> [B][T * Hq][d], row t * Hq + h
        self.q = q.reshape(q.shape[0], -1, q.shape[-1]) if q.ndim == 4 else q
        self.Kg = _f64(inputs.get("Kg"))
        self.Vg = _f64(inputs.get("Vg"))
        self.Kmg = _f64(inputs.get("Kmg"))
        self.P = _f64(inputs.get("P"))
        self.Kp = _f64(inputs.get("Kp"))

    def kv_rows(self, bk: int, g: int, rows: np.ndarray):
        idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=self._K.device)
        Kr = self._K[bk, g].index_select(0, idx)
        Vr = self._V[bk, g].index_select(0, idx)
        return _f64(Kr), _f64(Vr)


class PrefillSource:
    """Inputs of one prefill step as the oracle reads them: Q [B][Hq][L][d] and K, V
    [B][Hkv][L][d] on any device; rows are widened to fp64 on demand."""

    def __init__(self, inputs: dict):
        self._Q, self._K, self._V = inputs["Q"], inputs["K"], inputs["V"]

    def _rows(self, t, b, h, rows):
        idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)
        return _f64(t[b, h].index_select(0, idx))

    def q_rows(self, b: int, h: int, rows) -> np.ndarray:
        return self._rows(self._Q, b, h, rows)

    def k_all(self, b: int, g: int) -> np.ndarray:
        return _f64(self._K[b, g])

    def kv_rows(self, b: int, g: int, rows):
        return self._rows(self._K, b, g, rows), self._rows(self._V, b, g, rows)


class GistPrefillSource:
    """Inputs of one gist-masked prefill step as the oracle reads them: raw Q [B][Hq][N][d],
    K, V [B][Hkv][N][d] and gist Qg [B][Hq][M][d], Kg, Vg [B][Hkv][M][d] on any device; rows are
    widened to fp64 on demand."""

    def __init__(self, inputs: dict):
        self._t = {k: inputs[k] for k in ("Q", "K", "V", "Qg", "Kg", "Vg")}

    def _rows(self, name, b, h, rows):
        t = self._t[name]
        idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=t.device)
        return _f64(t[b, h].index_select(0, idx))

    def q_row(self, b: int, h: int, kind: str, i: int) -> np.ndarray:
        return self._rows("Q" if kind == "raw" else "Qg", b, h, [i])[0]

    def raw_kv_rows(self, b: int, g: int, rows):
        return self._rows("K", b, g, rows), self._rows("V", b, g, rows)

    def gist_kv_rows(self, b: int, g: int, rows):
        return self._rows("Kg", b, g, rows), self._rows("Vg", b, g, rows)
