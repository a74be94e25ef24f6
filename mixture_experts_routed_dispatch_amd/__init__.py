"""MI355X (gfx950) routed Mixture-of-Experts expert layer.

Importing this package touches no GPU: the HIP library is loaded on first use
by :mod:`mixture_experts_routed_dispatch_amd.moe`.
"""
