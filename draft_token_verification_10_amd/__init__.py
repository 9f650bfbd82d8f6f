"""libspecverify: the speculative-decoding verification step on AMD Instinct
MI355X (gfx950), as a C-ABI shared library with a thin ctypes binding.

``binding`` loads ``libspecverify.so`` (built by ``__graft_entry__.build()``)
and exposes ``sv_verify_greedy``, ``sv_verify_stochastic``,
``sv_workspace_bytes`` and ``sv_status_string`` on torch ROCm tensors.
``workloads`` draws the seeded synthetic inputs.
"""
