"""DSA forward hot path on MI355X (gfx950): lightning indexer, top-k select
and sparse MQA attention, as hand-written HIP kernels behind a C ABI.

The Python side only marshals arguments (`binding`) and draws seeded
synthetic inputs (`inputs`)."""
