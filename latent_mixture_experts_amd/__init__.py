"""latent_mixture_experts_amd: the latent mixture-of-experts layer of the
Edge0 145B / 120B models on AMD Instinct MI355X (gfx950).

The compute lives in ``liblmoe.so`` (hand-written HIP, C ABI declared in
``include/lmoe.h``). ``lmoe`` is its thin ctypes binding; ``workloads`` draws
seeded synthetic inputs. Importing this package does not load the library.
"""

__all__ = ["lmoe", "workloads"]
