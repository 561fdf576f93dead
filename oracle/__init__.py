"""CPU oracle for the FP4 weight-only MoE expert path (test infrastructure).

This package is the plain, slow, obviously correct definition of what the GPU
path computes.  It is test infrastructure: only the tests, the smoke check
and the CPU-baseline leg of the benchmark may import it.  The product path
(the HIP library and its Python binding) never imports, calls or links it,
and it shares no code with that path.

It holds two independent definitions: the numpy float64 modules below, and
a plain single-threaded C++17 float64 oracle (qmoe_oracle.cpp, loaded by
cpp.py through ctypes) that shares no code with them.  Every function cites
the passage of the pages it follows:

  * "[CUDA] Speed up the NVFP4 QMoE decode GEMV and enable it for MTP verify"
    (onnxruntime PR 31159) -- the decode GEMV, expanded rows up to 64;
  * "[CUDA] Coalesce QMoE MXFP4/NVFP4 weight dequantization" (PR 31349) --
    the dequant kernel and its codecs;
  * "MoE and QMoE -- CUDA Operator Documentation" (sections 1, 6.5, 8, 9b, 13);
  * "[CUDA] Add an opt-in FP8 DeepGEMM MoE decode path for QMoE" (PR 32122);
  * "[CUDA] Cut the MoE routing prologue/epilogue cost for small-batch
    decode" (PR 31156) -- top-k with a stable key, expert maps, finalize.

Modules: codecs (E2M1, E4M3FN, E8M0, bfloat16 rounding), dequant, route
(softmax top-k and expert maps), moe (FC1+SwiGLU, FC2, finalize, layer),
tolerance (the floating-point comparison rule), cpp (the C++ oracle: the
same steps, same call names as route / moe).
"""
