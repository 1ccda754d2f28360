"""The two-term decode-step model (test and report infrastructure only).

"When quantization pays -- and when it does not" models one decode step as a
memory pipe and a math pipe that overlap: the step takes the longer of
  * streaming the weights:            W * b_w / beta
  * issuing the math plus conversion: 2 * W * B / P + W * c / D
where W is the number of streamed parameters, b_w the bytes per stored weight,
beta the HBM bandwidth, B the batch, P the peak of the tensor-core instruction
actually issued, c the non-tensor instructions per weight spent converting it
and D the non-tensor issue rate (sections "Model one decode step..." and
"The three regimes").  The page's equation itself did not survive extraction;
the form above is rebuilt from the surrounding definitions and is pinned by
reproducing every number the page prints (tests/golden/decode_model_h100.txt).
Weight-and-activation 8-bit schemes halve both terms (P doubles, c = 0).
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Machine:
    beta: float      # HBM bytes/s
    p_bf16: float    # dense bf16 tensor/matrix flop/s
    p_fp8: float     # dense fp8 flop/s
    d_valu: float    # non-tensor lane-instructions/s


# The page's card: H100 SXM, 3.35 TB/s, 989.4 TFLOP/s bf16, FP32 vector
# 67 TFLOP/s counted as 33.5e12 FMA lane-instructions/s.
H100_SXM = Machine(beta=3.35e12, p_bf16=989.4e12, p_fp8=2 * 989.4e12, d_valu=33.5e12)

# MI355X datasheet values: 8 TB/s HBM3E, 2.5 PFLOP/s dense bf16, 5.0 fp8,
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3e12 VALU lane-instructions/s.
MI355X = Machine(beta=8.0e12, p_bf16=2.5e15, p_fp8=5.0e15, d_valu=256 * 4 * 16 * 2.4e9)

B_BF16 = 2.0
B_INT8 = 1.0
B_INT4_G128 = 4.125 / 8.0     # 0.515625 bytes per stored weight
C_MARLIN = 2.0                # 8 non-tensor instructions per 4 weights


def step_bf16(W, B, m=H100_SXM):
    return max(W * B_BF16 / m.beta, 2.0 * W * B / m.p_bf16)


def step_w8a8_fp8(W, B, m=H100_SXM):
    return max(W * B_INT8 / m.beta, 2.0 * W * B / m.p_fp8)


def step_w4a16(W, B, c=C_MARLIN, m=H100_SXM):
    return max(W * B_INT4_G128 / m.beta, 2.0 * W * B / m.p_bf16 + W * c / m.d_valu)


def dequant_tax(W, c=C_MARLIN, m=H100_SXM):
    return W * c / m.d_valu


def w4a16_own_ridge(c=C_MARLIN, m=H100_SXM):
    """B where the W4A16 math term reaches its own memory floor."""
    return (B_INT4_G128 / m.beta - c / m.d_valu) * m.p_bf16 / 2.0


def m_star(m=H100_SXM):
    """The same ridge with the conversion assumed free."""
    return B_INT4_G128 / m.beta * m.p_bf16 / 2.0


def bf16_ridge(m=H100_SXM):
    return B_BF16 / m.beta * m.p_bf16 / 2.0


def w4a16_stops_paying(c=C_MARLIN, m=H100_SXM):
    """B where the W4A16 math term reaches the bf16 memory floor."""
    return (B_BF16 / m.beta - c / m.d_valu) * m.p_bf16 / 2.0


def w4a16_vs_fp8(c=C_MARLIN, m=H100_SXM):
    """B where the W4A16 math term reaches the 8-bit memory floor."""
    return (B_INT8 / m.beta - c / m.d_valu) * m.p_bf16 / 2.0
