"""paged_kv_attention_17_amd -- paged KV-cache attention for MI355X (gfx950)."""
