"""fp64 CPU oracle for Flex-Flash-Attention (test infrastructure only)."""
