"""Plain CPU oracle (test infrastructure only)."""
