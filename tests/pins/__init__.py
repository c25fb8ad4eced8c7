"""Independent references used only to pin the CPU oracle."""
