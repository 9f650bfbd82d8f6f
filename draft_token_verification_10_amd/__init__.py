"""libspecverify: the speculative-decoding verification step on AMD Instinct
MI355X (gfx950), as a C-ABI shared library with a thin ctypes binding.

``binding`` loads ``libspecverify.so`` (built by ``__graft_entry__.build()``)
and exposes its entry points on torch ROCm tensors: ``sv_verify_stochastic``,
``sv_verify_greedy``, their ``_ragged`` forms, ``sv_sample``,
``sv_verify_greedy_tree``, ``sv_commit``, ``sv_workspace_bytes`` and
``sv_status_string``.
``workloads`` draws the seeded synthetic inputs.
"""
