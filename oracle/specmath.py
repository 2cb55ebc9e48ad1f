"""Specified binary32 exp / sigmoid / SiLU (oracle; test infrastructure only).

Routing by "sigmoid affinity, then top-K" ([DSV3-MOE]) turns floating point
into an integer decision (which experts win), and SwiGLU's output is FP8
quantised ([DSV3-FP8]).  For those integers to agree bit for bit, both
implementations evaluate the sigmoid with the *same* sequence of IEEE binary32
operations.  This module is that sequence written for numpy float32 arrays;
the GPU library carries its own independent implementation of the same
written specification.

Specification (reading; the pages define no sigmoid algorithm).  Every
operation below is one correctly rounded binary32 operation; there is no fused
multiply-add:

  E(y):  y <- min(max(y, -80), 80)
         n <- rint(y * LOG2E)                      (round half to even)
         r <- (y - n * LN2_HI) - n * LN2_LO        (Cody & Waite, 1980)
         p <- c7; p <- p * r + c_k for k = 6 .. 0  (Horner, c_k = fl32(1/k!))
         E <- p * 2^n                              (exact power-of-two scaling)
  sigmoid(x) = 1 / (1 + E(-x))
  silu(x)    = x * sigmoid(x)

LN2_HI is ln 2 rounded to binary32 with its 9 lowest significand bits cleared,
so n * LN2_HI is exact for |n| <= 2^7; LN2_LO = fl32(ln 2 - LN2_HI).  With
|y| <= 80 the factor 2^n stays a normal number and so does the result.
The truncated Taylor series has relative error below 6e-9 on
|r| <= ln(2)/2, well under half an ulp; the rounding of the Horner steps keeps
the total within a few ulp of exp, which the tests check.
"""

import math

import numpy as np

F32 = np.float32

LOG2E = F32(1.0 / math.log(2.0))
_LN2_F32_BITS = np.array([math.log(2.0)], dtype=np.float32).view(np.uint32)[0]
LN2_HI = np.array([_LN2_F32_BITS & np.uint32(0xFFFFFE00)], dtype=np.uint32).view(np.float32)[0]
LN2_LO = F32(math.log(2.0) - float(LN2_HI))
TAYLOR = [F32(1.0 / math.factorial(k)) for k in range(8)]
CLAMP = F32(80.0)


def spec_exp(y):
    """E(y) of the specification above, elementwise on float32."""
    y = np.asarray(y, dtype=np.float32)
    y = np.minimum(np.maximum(y, -CLAMP), CLAMP)
    n = np.rint(y * LOG2E)
    r = (y - n * LN2_HI) - n * LN2_LO
    p = np.full_like(r, TAYLOR[7])
    for k in range(6, -1, -1):
        p = p * r + TAYLOR[k]
    two_n = ((n.astype(np.int32) + 127) << 23).astype(np.int32).view(np.float32)
    return (p * two_n).astype(np.float32)


def spec_sigmoid(x):
    """sigmoid(x) = 1 / (1 + E(-x)) in binary32, as specified above."""
    x = np.asarray(x, dtype=np.float32)
    return (F32(1.0) / (F32(1.0) + spec_exp(-x))).astype(np.float32)


def spec_silu(x):
    """silu(x) = x * sigmoid(x) in binary32 (the SwiGLU activation)."""
    x = np.asarray(x, dtype=np.float32)
    return (x * spec_sigmoid(x)).astype(np.float32)
