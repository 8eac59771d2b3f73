"""fp64 CPU oracle for AB-Attention sampled block-sparse attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this package:
only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
it. It shares no code with the HIP library and does not import it.

Sources. Two web pages describe the method:
  * edumints blog, "AB-Attention: Video Difuzyon Transformer'larini
    Hizlandirmak Icin Dogru Blok Dikkat Mekanizmasi" (cited below as [edumints]),
    sections "attention bottleneck", "three innovations", "results";
  * hamidun news, "AB-Attention speeds up video generation up to 2.23x and
    skips 92% of attention compute" (Arabic; cited as [hamidun]), sections
    "where earlier sparse schemes fail", "three techniques in AB-Attention"
    (paragraphs on IBCS, SIP and the kernel), "how it was measured".
No page prints a formula, listing or worked number, so every concrete choice
below is a reading of their prose; each reading is stated where it is made.

Steps, in the order the method applies them, and what pins each:

  mean_keys           [hamidun, three techniques, IBCS]   closed form; pinned
  kmeans_block        [hamidun, IBCS; edumints, three innovations]  pinned by
                      invariants, C=1 block mean, C=n self-clusters, planted
                      clusters and a hand-worked example
  kmeans_tie_variants the same iteration with near-tie decisions taken the
                      other way (test aid); pinned by a hand-worked exact tie
  ibcs_scores_row     [hamidun, IBCS]                      pinned by C=1 and C=n
                      reductions to library softmax, invariants, hand example
  sip_probabilities   [hamidun, SIP; edumints, three innovations]  pinned by
                      hand-worked examples and invariants
  philox4x32_10       published counter-based generator (Salmon et al. 2011)
                      pinned by its published known-answer values
  sip_draw_row        [hamidun, SIP]                       pinned by inclusion
                      frequencies over many seeds
  systematic_draw_row fixed-size design (reading of the pages' fixed budget)
                      pinned by exact inclusion counts over a grid of U,
                      the closed form for equal sizes, always-taken p = 1
                      blocks and the sample size
  ht_attention_row    [hamidun, SIP and kernel paragraphs] pinned by budget 100%
                      == dense, "p = 25% counts four times" == physical key
                      duplication through library attention, Monte-Carlo
                      unbiasedness of numerator and normaliser
  dense_attention     textbook softmax attention; pinned against the library
                      scaled-dot-product attention on the CPU
"""
from .ibcs import (mean_keys, kmeans_block, kmeans_tie_variants, ibcs_scores_row, ibcs_row,
                   query_rows)
from .sip import (sip_probabilities, sip_draw_row, sip_uniforms, fixed_point_scores,
                  systematic_uniform, systematic_sizes, systematic_select,
                  systematic_draw_row, draw_row)
from .philox import philox4x32_10
from .attention import (ht_attention_row, dense_attention, dense_attention_rows,
                        ht_numerator_denominator)
from .plan import build_plan, plan_from_scores, ibcs_scores, plan_attention, OraclePlan

__all__ = [
    "mean_keys", "kmeans_block", "kmeans_tie_variants", "ibcs_scores_row", "ibcs_row", "query_rows",
    "sip_probabilities", "sip_draw_row", "sip_uniforms", "fixed_point_scores",
    "systematic_uniform", "systematic_sizes", "systematic_select", "systematic_draw_row",
    "draw_row",
    "philox4x32_10", "ht_attention_row", "dense_attention", "dense_attention_rows",
    "ht_numerator_denominator", "build_plan", "plan_from_scores", "ibcs_scores",
    "plan_attention", "OraclePlan",
]
