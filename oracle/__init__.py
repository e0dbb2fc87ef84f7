"""CPU oracle of the DSA forward path (float64 NumPy).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library.
"""
from .dsa_oracle import (OracleInputs, decode_bf16, decode_e4m3fn, decode, E4M3FN_TABLE,
                         sequence_of, candidate_count, gather_rows, index_scores,
                         query_index_operands, query_index_scores, topk, topk_padded,
                         sparse_mla, query_attention, forward, E4M3FN_MAX, encode_e4m3fn, quantize_fp8,
                         append_index_keys, dense_attention, dense_forward,
                         attention_distribution, kl_rows, index_scores_backward, indexer_kl_loss,
                         sparse_mla_backward, sparse_attention_backward, sparse_attention_distribution,
                         sparse_indexer_kl_loss)

__all__ = ["OracleInputs", "decode_bf16", "decode_e4m3fn", "decode", "E4M3FN_TABLE",
           "sequence_of", "candidate_count", "gather_rows", "index_scores",
           "query_index_operands", "query_index_scores", "topk", "topk_padded", "sparse_mla",
           "query_attention", "forward", "E4M3FN_MAX", "encode_e4m3fn", "quantize_fp8", "append_index_keys",
           "dense_attention", "dense_forward",
           "attention_distribution", "kl_rows", "index_scores_backward", "indexer_kl_loss",
           "sparse_mla_backward", "sparse_attention_backward", "sparse_attention_distribution",
           "sparse_indexer_kl_loss"]
