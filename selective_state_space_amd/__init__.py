"""MI355X-native selective state-space scans (placeholder; binding follows)."""
