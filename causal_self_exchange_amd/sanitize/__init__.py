"""Host-only sanitizer build of the C API (argument checks, workspace
queries, status strings, kernel selection) for the ABI tests."""
