// matrix-core chunked prefill (next)
