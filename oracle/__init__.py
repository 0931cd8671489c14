"""fp64 CPU oracle for the ReplaySSM decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call, link or run anything in this package.  The
product (``ssm_layer_decode_amd``) never does; this package never imports the
product either.  The two share no code: the only thing both sides consume is
the seeded inputs drawn by ``ssm_layer_decode_amd.workloads``, handed over as
plain arrays by the tests.

Citation keys (sources are web pages describing one method):
  [ru] aikraft.ru, "ReplaySSM: Революция в декодировании гибридных моделей",
       sections 01-07.
  [ar] sitech.ge, "NVIDIA و Dao AI Lab يقدّمان ReplaySSM لتسريع فك ترميز النماذج
       الهجينة", sections "how ReplaySSM works", "reducing state traffic and
       simplifying rollback", "limiting quantization error".
  [zh] ai.cheesepanini.fun knowledge card "ReplaySSM——重新思考混合模型解码的状态存储",
       sections "method points", "main results", "limitations".
Equation names used throughout:
  eq.R   the scalar-decay recurrence  S_t = a_t S_{t-1} + v_t k_t^T,  o_t = S_t q_t
         ([ru] §01).
  eq.U   its unrolled window  S = g_h S_ckpt + sum_j g_{j+1:h} v_j k_j^T
         ([ru] §03; [zh] method points).
  eq.O1  output-only rank-1 form  o = (v k^T) q = v (k^T q)  ([ru] §05).
  eq.OT  output-only T-query chunk  O = S_ckpt Q D + V (W ⊙ K^T Q)  ([zh] method
         points).

Modules:
  recurrence  eq.R stepped one token at a time in fp64 (decode and speculative
              verify/commit); the plain definition ReplaySSM must reproduce.
  exact       rational (Fraction) eq.R and eq.U for brute-force pins.
  bookkeeping integer model of the record buffer and its pointer.
  quant       bf16 and OCP fp8 e4m3fn encoders written from the format
              definitions, and the per-row scaled quantiser.
  lowprec     the split-precision read path and the fully quantised arm.
  cpu_c       ctypes front of the plain C fp64 stepper (OpenMP over independent
              (sequence, head) pairs) used for large sizes and CPU timing.

Parity status per function is stated in each module's header.
"""
