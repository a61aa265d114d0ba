"""MI355X (gfx950) latent-MoE layer tail: router top-k + permutation, FP8 /
MXFP4 routed-expert grouped GEMMs, combine + RMSNorm, BF16 up-projection with
the BF16 shared-expert output added in FP32.  The compute lives in the HIP
library ``libmoe_tail.so`` behind the C ABI of ``include/moe_tail.h``;
``binding`` is its ctypes front end."""
