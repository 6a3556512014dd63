"""pytest plugin for the sanitizer run: points the oracle and the binding at the sanitized
builds named by GDN_SAN_ORACLE and GDN_SAN_LIBGDN before any test loads a library."""
import os


def pytest_configure(config):
    import oracle
    from gated_deltanet_recurrent_02_amd import _binding
    oracle.LIBRARY = os.environ["GDN_SAN_ORACLE"]
    _binding.LIBRARY = os.environ["GDN_SAN_LIBGDN"]
