"""pytest plugin for the AddressSanitizer run of the CPU tier: points the
binding at the host-only ASan build of the C-ABI layer and the oracle wrapper
at the ASan build of the oracle (paths from KDA_ASAN_HOST_LIB and
KDA_ASAN_ORACLE_LIB, set by tests/test_host_asan.py)."""
import os


def pytest_configure(config):
    from linear_attention_recurrence_11_amd import binding
    import oracle.build

    host = os.environ["KDA_ASAN_HOST_LIB"]
    binding.library_path = lambda: host
    binding._LIB = None
    oracle.build.LIB = os.environ["KDA_ASAN_ORACLE_LIB"]
