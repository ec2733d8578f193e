"""MI355X-native tree-verify MLA for DDTree speculative decoding."""
