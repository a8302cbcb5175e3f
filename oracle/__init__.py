"""fp64 CPU oracle for LLA latent-store decode. Test infrastructure only: imported by
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg, never by
the product path."""
