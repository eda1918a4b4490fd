"""Imbalance metric (test infrastructure only).

[MoonEP-news] "MoonEP 针对的问题": maxvio = max_e (T_e / T_bar) - 1, where
T_e is the number of tokens routed to expert e and T_bar the count each
expert would get under perfect balance, here R*S*K / E.  maxvio = 0 means
perfect balance; since T_e <= R*S (K distinct experts per token) maxvio is at
most E/K - 1.

Pinned by tests/test_oracle_plan.py: perfectly uniform routing gives 0, all
tokens on the same K experts gives E/K - 1.
"""
import numpy as np


def maxvio(counts, R, S, K):
    T = np.asarray(counts, np.float64)
    tbar = R * S * K / T.size
    return float(T.max() / tbar - 1.0)
