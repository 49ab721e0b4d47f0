"""Tree masks for the tree-draft tests: the generator lives with the other
seeded inputs in ``workloads``."""
from workloads import tree_masks  # noqa: F401
