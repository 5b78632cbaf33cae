"""Test-only native helpers (built by __graft_entry__.build())."""
