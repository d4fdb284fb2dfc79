"""CPU oracle for the speculative KV coder -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow reference that the HIP library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it; the product path (``entropy_coding_amd``)
never imports, calls or links anything here, and the two share no code.

Sources: the wiki page "Speculative KV Coding" (aisparkup.com) and the blog
post "推测性KV编码：用预测模型实现缓存无损压缩4倍" (blog.hotdry.top).  The pages
fix the model (a three-part mixture around a predictor mean) and the claim
(lossless, size close to the model's cross-entropy); they do not fix the coder,
so every integer detail below follows the written format KVC-1 whose readings
are listed, with the passages they rest on, in the design notes.

Parity status of each function (what pins it other than itself):
  order_index / bits_of_order  -- brute force over every bit pattern, torch's
                                  own bf16 / float8_e4m3fn decoders
  boundary_positions           -- exact midpoint identity in float64
  phi_tables / mixture_table  -- scipy.special.ndtr, symmetry, closed values,
                                  the wide table against the narrow one at z/3
  h_fx / cdf                   -- invariants (C(0)=0, C(N)=M, f>=1) and the
                                  continuous mixture within a derived bound
  gauss_cum / escape_cum       -- the slot ranges tile the coder range and
                                  add up to the mixture frequencies
  encode / decode              -- round trip, exact size band, unbounded
                                  big-integer rANS, a two-token chunk whose
                                  payload (states, word order of every step
                                  block, padding) is written out with Python
                                  ints from the format's steps
  build_marginal               -- brute-force counting on tiny inputs
  calibrate_sigma              -- float64 closed form, minimum of the
                                  Gaussian cost
  side_hash                    -- splitmix64's published outputs for seed 0
                                  pin the mixer; a small case summed word by
                                  word with Python ints pins the sum
  model_bits_float             -- closed forms for the narrow part alone and
                                  the wide part alone (a Gaussian at 3 sigma)
                                  in a constant-ulp region; the escape part
                                  alone against the smoothed histogram counted
                                  pattern by pattern
  split_budgets / h_fx_lanes   -- (per-channel split, S-14) chunks whose lanes
                                  share one weight equal the global-weight
                                  chunks byte for byte; each lane's final
                                  state and word count from a one-lane rANS
                                  written out with Python ints; code lengths
                                  per channel
  calibrate_split              -- a float64 brute force over the candidates
  sigma_blocks / calibrate_sigma with blocks (S-11)
                               -- one block over every token and equal blocks
                                  reproduce the per-plane payloads; per-block
                                  closed form of the calibration
  log2_table_q16 / code_len_q16 / calibrate_sigma_rate (S-12)
                               -- log2 (exact at powers of two, high by less
                                  than 0.0056 bits); a float64 brute force of
                                  the exact code length over the candidates
  student_t_cdf_mp / narrow_table (S-13)
                               -- scipy's stdtr for nu = 1..16, the closed
                                  forms for nu = 1, 2; the float model of data
                                  drawn from the truncated t against its
                                  closed-form entropy
  crc32 / stream_header / parse_header
                               -- zlib's crc32 and the standard check value;
                                  every damaged field refused
  model_bits_int               -- the coded size: payload minus the model's
                                  bits within the coder's bounds per lane
  scatter_to_pages             -- plain loops over every (plane, token)
  published bits/scalar of the pages (6.74..5.92, 2.05-2.59)
                               -- parity unpinned: needs Qwen3 weights and C4
"""

from .kvc_oracle import *  # noqa: F401,F403
