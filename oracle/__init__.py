"""Test-only CPU oracle (fp64 direct loops).  See oracle/oracle.py."""
