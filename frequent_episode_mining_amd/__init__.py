"""MI355X-native serial-episode counting (binding is added with the HIP library)."""
