"""Low-bit weight x activation product with the rotation applied online.
Test infrastructure only.

[HARP] 1 and 2.4: the weights are quantised in the rotated basis (RHT, then
low-bit codes) and the rotation is applied to the activations at inference,
by fused kernels with O(d log d) cost.  The product a layer computes is
y = x W_hat^T, W_hat the dequantised weight brought back by the inverse RHT:
W_hat[o] = S Hn (q[o] * s[o]) (rtn.dequantize_inverse).  Written out here as
that definition: dense W_hat, then the plain product.
"""

import numpy as np

from .rtn import dequantize_inverse


def rht_gemv(x, codes, s16, s, bits, group, n):
    """y[t, o] = sum_i x[t, i] W_hat[o, i], fp64; x [tokens, n]."""
    w_hat = dequantize_inverse(codes, s16, s, bits, group, n)
    return np.asarray(x, dtype=np.float64) @ w_hat.T
