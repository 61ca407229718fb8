"""fp4q: MI355X-native FP4 compression of tensor-parallel communication."""
