"""Constants of the quantization scheme, as the oracle reads them.

The pages fix none of these (they say only "low-bit", podcast notes section
"02:48 There were clearly faster compute units on the hardware").  They are
the library's stated design; the HIP side defines its own copies and a test
checks that both agree.
"""

BQ = 128          # query tokens per Q scale block
BK = 64           # key tokens per K scale block; also the softmax chunk length
VB = 32           # key tokens per V (FP8 mode) E8M0 scale block
QMAX = 127        # symmetric INT8 range [-127, 127]
F8MAX = 448.0     # largest finite OCP e4m3fn value
KMEAN_CHUNK = 128  # tokens per first-level partial sum of the K mean
TAU = 4.0         # lazy running-max threshold, in log2 units
PSHIFT_FP8 = 4    # P is stored as e4m3(p * 2^4) in FP8 PV mode
PSHIFT_16 = 0     # no pre-scale when P is rounded to fp16/bf16
LOG2E = 1.4426950408889634

PV_16 = 0
PV_FP8 = 1
PV_AUTO = 2      # per (b,h): FP8 unless channel balance moved a channel (quant.pv_modes_auto)

__all__ = ["BQ", "BK", "VB", "QMAX", "F8MAX", "KMEAN_CHUNK", "TAU",
           "PSHIFT_FP8", "PSHIFT_16", "LOG2E", "PV_16", "PV_FP8", "PV_AUTO"]
