"""CPU oracle for context-parallel attention: plain, slow, float64.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The product library (``context_attention_dit_amd``) never imports it,
and it imports nothing from the product: the two share no code, only the
seeded inputs of the ``synthetic`` package.

Functions and the passages they follow:
  attention.attention       full softmax attention + LSE by brute force
                            (diffusers Context parallelism guide, Ring Attention;
                            Ulysses SP article, notes 2 and 7 for causal masking
                            from positions)
  attention.chunk_partial   one ring hop's (O_c, LSE_c)
                            (diffusers parallel API, ContextParallelConfig:
                            convert_to_fp32 output + LSE)
  attention.lse_merge       closed-form merge of partials
                            (SGLang Diffusion Sequence Parallelism, Numerics
                            across node boundaries)
  attention.ring_attention  ring order of hops, then merge (diffusers guide,
                            Ring Attention and Ring Anything Attention)
  relayout.seq2head / head2seq (and *_loop forms)
                            Ulysses sequence<->head regrouping (diffusers guide,
                            Ulysses Attention; Ulysses SP article, notes 3-4)
  relayout.seq2head_vt (and seq2head_vt_loop)
                            seq2head of V delivered key-contiguous per head
  relayout.anything_seq2head / anything_head2seq (and *_loop forms)
                            the same with uneven per-rank token and head counts
                            (diffusers guide, Ulysses Anything Attention)
  relayout.kv_gather (and kv_gather_loop; kv_gather_vt: V key-contiguous)
                            the K/V all-gather's unpack (SGLang Diffusion
                            Sequence Parallelism, Choosing The Attention
                            Exchange: kv_gather)
  backward.attention_grad   dQ, dK, dV of full attention by the chain rule
  backward.backward_delta   Delta_i = <dO_i, O_i>
  backward.chunk_grad       one K/V chunk's share of the backward from the saved
                            LSE and Delta (Ulysses SP article: training with long
                            contexts, notes 2: no stored score matrix; diffusers
                            guide, Ring Attention, for the chunk decomposition)

Every function is pinned in ``tests/test_oracle.py`` and
``tests/test_oracle_backward.py`` against closed forms,
hand-derived golden values (``tests/golden/``), identities, a library
routine (torch's fp64 scaled_dot_product_attention, and its autograd for the
backward), finite differences and explicit loops.
"""
from .attention import (attention, bf16_bits_to_f64, chunk_partial,
                        lse_merge, ring_attention, softmax_matrix)
from .backward import attention_grad, backward_delta, chunk_grad
from .relayout import (anything_head2seq, anything_head2seq_loop, anything_seq2head,
                       anything_seq2head_loop, even_split, head2seq, head2seq_loop, kv_gather,
                       kv_gather_loop, kv_gather_vt, seq2head, seq2head_loop, seq2head_vt,
                       seq2head_vt_loop)

__all__ = ["attention", "chunk_partial", "lse_merge", "ring_attention", "softmax_matrix",
           "bf16_bits_to_f64", "seq2head", "head2seq", "seq2head_loop",
           "head2seq_loop", "seq2head_vt", "seq2head_vt_loop", "anything_seq2head",
           "anything_head2seq", "anything_seq2head_loop",
           "anything_head2seq_loop", "even_split", "kv_gather", "kv_gather_loop", "kv_gather_vt",
           "attention_grad", "backward_delta", "chunk_grad"]
