"""Comparison metrics.  Test infrastructure.

jepa.cpp Quantization page, "How the accuracy was measured": per-token
cosine (mean and worst token), rel_max = max|a - b| / max|b| and
rel_fro = ||a - b|| / ||b||.  The LeVJEPA card's "Files" table reports the
mean, median and worst per-token cosine.
"""
from __future__ import annotations

import numpy as np


def token_cosines(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Cosine of each row (token) of a against the same row of b, in float64."""
    a = np.asarray(a, dtype=np.float64).reshape(-1, a.shape[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, b.shape[-1])
    num = np.sum(a * b, axis=1)
    den = np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1)
    return num / den


def rel_max(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def report(a: np.ndarray, b: np.ndarray) -> dict:
    """a = result under test, b = oracle."""
    c = token_cosines(a, b)
    return dict(cos_mean=float(np.mean(c)), cos_median=float(np.median(c)),
                cos_worst=float(np.min(c)), rel_max=rel_max(a, b), rel_fro=rel_fro(a, b))
