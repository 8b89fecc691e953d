"""MI355X-native dense-transformer prefill: a C-ABI HIP library (libtf_prefill.so) and a
thin torch-facing binding. Every step of the forward runs in the library's kernels."""
from ._abi import KERNEL_CLASSES, TfError, load  # noqa: F401
from .model import PrefillModel, quantize_q8_0, upload_weights  # noqa: F401
