"""relative_bias_gqa_amd: relative-bias GQA attention for MI355X (placeholder; binding lands with the HIP library)."""
