"""MI355X-native audio prefill KV-cache compression (scores -> spectral score
smoothing -> head-aware budget -> top-k -> gather), behind the C ABI of
include/kvc.h.  The HIP library is loaded on first use."""
