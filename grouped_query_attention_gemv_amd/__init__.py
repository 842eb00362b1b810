"""MI355X grouped-query attention block (Llama 3.1 8B shapes)."""
