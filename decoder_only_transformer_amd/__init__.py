"""MI355X (gfx950) Llama 2 decoder forward: prefill + KV-cache decode behind a C ABI.

`abi` is the ctypes binding of include/llama_mi355x.h (same names as the C entry points);
`runtime` keeps weights and workspace in torch device memory and drives the generate
schedule; `build_lib` compiles the HIP library in-tree.
"""
from . import abi  # noqa: F401
