"""Error bars of the parity tests (no GPU or torch needed to import).

Outputs: max relative row error 1e-4 for fp32 paths and 2e-2 for bf16 paths.

Gradients of the bf16 backward, entry by entry against the root-sum-square
R of the entry's terms (oracle "rss_<name>": the gradient written out as one
sum of products of leaf factors). Each term reaches the GPU's sum through at
most four roundings to bf16, each a relative error of at most u = 2^-8 and
close to uniform: dO, which also carries the bf16 P of the recomputed
forward; P or dS as an MFMA operand; and the returned value. Independent
errors of spread u / sqrt(3) each give an error of spread at most
sigma = u sqrt(4 / 3) R, about 1.15 u R, whatever the signs of the terms.
Over at most 10^7 entries a Gaussian stays below 5.7 sigma; the bar 8 u is
about 7 sigma (a false alarm about once in 3 * 10^4 runs of 10^7 entries).
The backward on the forward's saved output (HSTU_FLAG_SAVED_FORWARD) adds
one rounding, the forward's bf16 deviations behind dO: five roundings,
sigma = u sqrt(5 / 3), about 1.29 u R, and the bar is about 6.2 sigma.
A term that is missing altogether costs about its own size; on random data
one 64-key tile of a row is a large part of R (a CPU pin shows such a dQ
scoring far above the bar).
"""
U_BF16 = 2.0 ** -8

TOL = {"f32": 1e-4, "bf16": 2e-2}

GRAD_RSS_BF16 = 8 * U_BF16
