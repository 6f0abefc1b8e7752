"""MI355X-native tiled online-softmax attention (prefill, split-KV decode,
merge, paged-KV gather) behind a C-ABI library of hand-written HIP kernels
for gfx950. The Python binding in :mod:`online_softmax_tiled_amd.api` only
marshals torch tensors to raw pointers and a stream; every step runs in the
library's kernels."""
