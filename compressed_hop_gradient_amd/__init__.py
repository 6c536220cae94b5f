"""DynamiQ hot path (variable-bitwidth gradient quantiser and fused
decompress-accumulate-recompress hop) for MI355X; see include/dq.h."""
