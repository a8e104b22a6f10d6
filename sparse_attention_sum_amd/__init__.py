"""libdsa: the DeepSeek Sparse Attention hot path (lightning indexer, top-k, sparse MLA) on MI355X."""
