"""MI355X-native DSpark sequential Markov draft-sampling step (placeholder;
the binding is added with the HIP library)."""
