// The pipelined prefill kernel with the fused input prologue (q/k L2 norm, beta sigmoid,
// g -softplus), compiled as a translation unit of its own from gdn_prefill_pipe.hip so
// that the plain kernel's code and register allocation are unaffected.
#define GDN_PIPE_PROLOGUE 1
#include "gdn_prefill_pipe.hip"
